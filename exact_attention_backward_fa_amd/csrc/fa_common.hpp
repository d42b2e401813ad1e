// Device-side helpers shared by the attention kernels (gfx950 / CDNA4).
//
// Matrix products use v_mfma_f32_32x32x16_{f16,bf16}: a 64-lane wave multiplies
// a 32x16 A tile by a 16x32 B tile into a 32x32 float32 tile.  Operand layout
// (lane = 0..63, l32 = lane % 32, g = lane / 32):
//   A: lane holds 8 16-bit values of row l32, at contraction slots 8g..8g+7;
//   B: lane holds 8 16-bit values of column l32, at the same slots;
//   C: lane holds 16 floats; element i is row 8*(i/4) + 4g + (i%4), column l32.
// Only the pairing of A's and B's slots matters to the product, so when an A
// operand is built from a C tile (P or dS feeding the next product) its slot e of
// k-step c stands for C row crow(c, g, e), and the B operand is loaded so that
// the same slot holds the same contraction index.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Row of a 32x32 C tile held in element i by lane group g.
__device__ __forceinline__ constexpr int crow_of(int i, int g) {
  return 8 * (i >> 2) + 4 * g + (i & 3);
}

// DT = 0: fp16, DT = 1: bf16.
template <int DT> struct Dt;

template <> struct Dt<0> {
  static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  // Two floats to two fp16 in one dword, round to nearest even.
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    f16x2 r = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, r);
  }
  static __device__ __forceinline__ float lo(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
  }
  static __device__ __forceinline__ float hi(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
  }
  static __device__ __forceinline__ uint16_t one(float x) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);
  }
};

template <> struct Dt<1> {
  static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    bf16x2 r = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, r);
  }
  static __device__ __forceinline__ float lo(uint32_t w) {
    return __builtin_bit_cast(float, w << 16);
  }
  static __device__ __forceinline__ float hi(uint32_t w) {
    return __builtin_bit_cast(float, w & 0xffff0000u);
  }
  static __device__ __forceinline__ uint16_t one(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
  }
};

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Pack elements 8c .. 8c+7 of a C tile into an A/B operand (slot e = element 8c+e).
template <int DT>
__device__ __forceinline__ u32x4 pack_c_slice(const f32x16& x, int c) {
  u32x4 r;
  r[0] = Dt<DT>::pack2(x[8 * c + 0], x[8 * c + 1]);
  r[1] = Dt<DT>::pack2(x[8 * c + 2], x[8 * c + 3]);
  r[2] = Dt<DT>::pack2(x[8 * c + 4], x[8 * c + 5]);
  r[3] = Dt<DT>::pack2(x[8 * c + 6], x[8 * c + 7]);
  return r;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16-byte global load/store helpers.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

__device__ __forceinline__ u32x4 zero_u4() {
  u32x4 z = {0u, 0u, 0u, 0u};
  return z;
}

// Store the 8 16-bit values of a 16-byte chunk, loaded from row r of a row-major
// tile at columns c0..c0+7, into a transposed LDS tile T[col][row] with row
// stride ldt (elements).
__device__ __forceinline__ void lds_store_transposed(uint16_t* T, int ldt, int r, int c0, u32x4 v) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    T[(c0 + 2 * j) * ldt + r] = (uint16_t)(v[j] & 0xffffu);
    T[(c0 + 2 * j + 1) * ldt + r] = (uint16_t)(v[j] >> 16);
  }
}

// B (or A) operand whose slots follow C rows crow(c, g, e) + base, read from a
// transposed LDS tile T[col][k] at column `col`.
__device__ __forceinline__ u32x4 lds_read_crow_operand(const uint16_t* T, int ldt, int col, int base,
                                                       int c, int g) {
  const uint16_t* p = T + col * ldt + base + 16 * c + 4 * g;
  u32x2 a = *reinterpret_cast<const u32x2*>(p);
  u32x2 b = *reinterpret_cast<const u32x2*>(p + 8);
  u32x4 r = {a[0], a[1], b[0], b[1]};
  return r;
}

}  // namespace fa
