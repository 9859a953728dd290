// Device-side helpers shared by the AlexNet HIP kernels (gfx950 / CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ax {

// bf16 values are stored as their 16-bit patterns.
typedef uint16_t bf16;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf2f(bf16 h) { return __uint_as_float((uint32_t)h << 16); }

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// float -> bf16, round to nearest, ties to even: gfx950's conversion
// instruction (v_cvt_pk_bf16_f32), one per pair in f2bf2.
__device__ __forceinline__ bf16 f2bf(float f) { return __builtin_bit_cast(bf16, (__bf16)f); }
// two floats -> a packed bf16 pair, a in the low half
__device__ __forceinline__ uint32_t f2bf2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// One SGD-with-momentum step on an element (paper form, lr inside v):
//   v <- mom * v - wd * lr * w - lr * g,   w <- w + v
// written with explicit fmas so that every kernel that applies it (the FC
// weight-gradient epilogue, the conv weight-gradient reductions and the bias
// update) rounds alike.
__device__ __forceinline__ void sgd_elem(float& w, float& v, float g, float mom, float wdlr, float lr) {
  v = fmaf(mom, v, -fmaf(lr, g, wdlr * w));
  w = w + v;
}

template <typename T> struct Num;
template <> struct Num<float> {
  static __device__ __forceinline__ float load(float v) { return v; }
  static __device__ __forceinline__ float store(float v) { return v; }
};
template <> struct Num<bf16> {
  static __device__ __forceinline__ float load(bf16 v) { return bf2f(v); }
  static __device__ __forceinline__ bf16 store(float v) { return f2bf(v); }
};

// 16-byte store marked non-temporal: the line is written back without being
// kept dirty in the last-level (Infinity) cache, so later streaming reads do
// not have to evict it first.  For data that is not read again soon.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void st_nt16(void* p, uint4 q) {
  __builtin_nontemporal_store((u32x4_t){q.x, q.y, q.z, q.w}, reinterpret_cast<u32x4_t*>(p));
}
__device__ __forceinline__ void st_nt16(void* p, float4 q) {
  st_nt16(p, make_uint4(__float_as_uint(q.x), __float_as_uint(q.y), __float_as_uint(q.z), __float_as_uint(q.w)));
}

// Eight consecutive elements of T as floats, from / to one or two 16-byte words.
template <typename T> struct Pack8;
template <> struct Pack8<bf16> {
  static __device__ __forceinline__ void load(const bf16* p, float* v) {
    const uint4 q = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  static __device__ __forceinline__ void store(bf16* p, const float* v) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = f2bf2(v[2 * i], v[2 * i + 1]);
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  }
  static __device__ __forceinline__ void store_nt(bf16* p, const float* v) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = f2bf2(v[2 * i], v[2 * i + 1]);
    st_nt16(p, make_uint4(w[0], w[1], w[2], w[3]));
  }
};
template <> struct Pack8<float> {
  static __device__ __forceinline__ void load(const float* p, float* v) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  static __device__ __forceinline__ void store(float* p, const float* v) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
  static __device__ __forceinline__ void store_nt(float* p, const float* v) {
    st_nt16(p, make_float4(v[0], v[1], v[2], v[3]));
    st_nt16(p + 4, make_float4(v[4], v[5], v[6], v[7]));
  }
};

// Pack V elements of T (16 bytes) into one 16-byte register word.
__device__ __forceinline__ uint4 pack_u4(const bf16 (&e)[8]) {
  return make_uint4((uint32_t)e[0] | ((uint32_t)e[1] << 16), (uint32_t)e[2] | ((uint32_t)e[3] << 16),
                    (uint32_t)e[4] | ((uint32_t)e[5] << 16), (uint32_t)e[6] | ((uint32_t)e[7] << 16));
}
__device__ __forceinline__ uint4 pack_u4(const float (&e)[4]) {
  return make_uint4(__float_as_uint(e[0]), __float_as_uint(e[1]), __float_as_uint(e[2]),
                    __float_as_uint(e[3]));
}

__device__ __forceinline__ void unpack_u4(uint4 q, bf16 (&e)[8]) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) { e[2 * i] = (bf16)(w[i] & 0xFFFFu); e[2 * i + 1] = (bf16)(w[i] >> 16); }
}
__device__ __forceinline__ void unpack_u4(uint4 q, float (&e)[4]) {
  e[0] = __uint_as_float(q.x); e[1] = __uint_as_float(q.y);
  e[2] = __uint_as_float(q.z); e[3] = __uint_as_float(q.w);
}

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of the
// multiply-xor bijection on a 128-bit counter with a 64-bit key that is bumped
// by the Weyl constants between rounds.
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
    const uint32_t lo0 = 0xD2511F53u * c.x, hi0 = __umulhi(0xD2511F53u, c.x);
    const uint32_t lo1 = 0xCD9E8D57u * c.z, hi1 = __umulhi(0xCD9E8D57u, c.z);
    c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
  }
  return c;
}

}  // namespace ax
