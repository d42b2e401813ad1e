// Device-side helpers shared by the attention kernels (gfx950 / CDNA4).
//
// The forward, dK/dV and dQ kernels multiply with v_mfma_f32_16x16x32 (layout
// below, Mx<DT>); the fused atomic kernel with v_mfma_f32_32x32x16_{f16,bf16}
// (Dt<DT>::mma): a 64-lane wave multiplies a 32x16 A tile by a 16x32 B tile into a
// 32x32 float32 tile.  Its operand layout (lane = 0..63, l32 = lane % 32,
// g = lane / 32):
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

#include <type_traits>
#include <utility>

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

// The 16x16x32 products (v_mfma_f32_16x16x32_{f16,bf16}) use, with l16 = lane % 16
// and j4 = lane / 16:
//   A: lane holds 8 16-bit values of row l16, at contraction slots 8*j4..8*j4+7;
//   B: lane holds 8 16-bit values of column l16, at the same slots;
//   C: lane holds 4 floats; element i is row 4*j4 + i, column l16.
// (Both layouts were checked on the GPU with an in-bounds probe.)

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
  static __device__ __forceinline__ f32x4 mma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
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
  // c + a.lo * b.lo + a.hi * b.hi (v_dot2c_f32_f16)
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
  }
};

template <> struct Dt<1> {
  static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
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
  // c + a.lo * b.lo + a.hi * b.hi (v_dot2c_f32_bf16)
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b),
                                           c, false);
  }
};

// MFMAs with explicit register placement.  With one wave per SIMD a kernel has
// 512 registers per lane: 256 VGPRs and 256 AGPRs.  The compiler, once a kernel
// may use more than 256, gives every MFMA an AGPR accumulator, which does not fit
// kernels whose long-lived accumulators alone fill the AGPRs.  These wrappers put
// the long-lived accumulators (dK, dV, dQ) in AGPRs ("a") and the short-lived
// score tiles in VGPRs ("v").  Being inline assembly, they are outside the
// compiler's hazard tracking, so the kernels keep at least one other MFMA between
// writing a tile and reading it from VALU code, and between producing an operand
// with VALU code and the MFMA that reads it; before the accumulators are read at
// the end, wait_mfma() lets the last MFMAs drain.
template <int DT> struct Mx;
template <> struct Mx<0> {
  static __device__ __forceinline__ f32x4 first16(const u32x4& a, const u32x4& b) {
    f32x4 d;
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
    return d;
  }
  static __device__ __forceinline__ void acc16(f32x4& c, const u32x4& a, const u32x4& b) {
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
  }
  // acc16 with a long-lived accumulator held in AGPRs
  static __device__ __forceinline__ void acc16a(f32x4& c, const u32x4& a, const u32x4& b) {
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
  }
  // first16 with the accumulator starting at c instead of zero
  static __device__ __forceinline__ f32x4 first16c(const u32x4& a, const u32x4& b, const f32x4& c) {
    f32x4 d;
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %3" : "=&v"(d) : "v"(a), "v"(b), "v"(c));
    return d;
  }
};
template <> struct Mx<1> {
  static __device__ __forceinline__ f32x4 first16(const u32x4& a, const u32x4& b) {
    f32x4 d;
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
    return d;
  }
  static __device__ __forceinline__ void acc16(f32x4& c, const u32x4& a, const u32x4& b) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
  }
  // acc16 with a long-lived accumulator held in AGPRs
  static __device__ __forceinline__ void acc16a(f32x4& c, const u32x4& a, const u32x4& b) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
  }
  // first16 with the accumulator starting at c instead of zero
  static __device__ __forceinline__ f32x4 first16c(const u32x4& a, const u32x4& b, const f32x4& c) {
    f32x4 d;
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %3" : "=&v"(d) : "v"(a), "v"(b), "v"(c));
    return d;
  }
};
// Enough idle issue cycles for any MFMA in flight to retire (a 32x32x16 MFMA is
// 8 passes of 4 cycles).
__device__ __forceinline__ void wait_mfma() {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

// wait_mfma() for a set of accumulators about to be read: the empty asm statements
// (ordered after the nops, as all volatile asm) tell the compiler the
// accumulators change there, so no read of them is scheduled before the wait.
template <int N0, int N1>
__device__ __forceinline__ void settle(f32x4 (&acc)[N0][N1]) {
  wait_mfma();
#pragma unroll
  for (int i = 0; i < N0; ++i) {
#pragma unroll
    for (int j = 0; j < N1; ++j) asm volatile("" : "+a"(acc[i][j]));
  }
}

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

__device__ __forceinline__ f32x4 zero4() {
  f32x4 z = {0.f, 0.f, 0.f, 0.f};
  return z;
}

// The four elements of a 16x16 C tile a lane holds (rows 4 j4 .. 4 j4 + 3 of its
// column), packed to 16 bits: half of a 16x16x32 A/B operand whose contraction
// runs along those rows.
template <int DT>
__device__ __forceinline__ u32x2 pack_c4(const f32x4& x) {
  u32x2 r = {Dt<DT>::pack2(x[0], x[1]), Dt<DT>::pack2(x[2], x[3])};
  return r;
}

// ---------------------------------------------------------------------------
// LDS tiles are row-major with rows of NG 16-byte granules (NG*8 16-bit columns)
// and no padding; granule j of row r is stored at position j ^ swz(r), so that
// both access patterns of the kernels avoid LDS bank conflicts:
//   - 16-byte row reads of an MFMA operand: 16 (16x16x32) or 32 (32x32x16)
//     consecutive rows at one logical granule;
//   - transposed reads (ds_read_b64_tr_b16): 4 consecutive rows x 32 bytes.
// For NG = 16 the XOR value takes row bits (r0, r2, r3, r1^r3) as granule bits
// 0..3; for NG = 8 it is row bits 1..3.  It was chosen by timing every invertible map whose granule bits are XORs
// of at most two row bits on an MI355X: it reads the 16x16x32 operand patterns at
// about 170 B/clk (rows) and 99 B/clk (transposed) per CU, and the 32x32x16 ones
// at 174 and 113, the best of all maps tried for both.
//
// SW selects the map: SW_MIN (the map above) or SW_LOWREG, an older map that reads
// the 32x32x16 patterns at the same rate (174 / 113 B/clk) and whose per-lane XOR
// values the compiler keeps in fewer registers; the fused atomic-dQ kernel, which
// is short of registers, uses it.
enum : int { SW_MIN = 0, SW_LOWREG = 1 };
template <int NG, int SW = SW_MIN>
__device__ __forceinline__ int swz(int r) {
  if (NG >= 16) {
    if (SW == SW_LOWREG) return ((r & 3) << 1) | ((r >> 2) & 1) | (((r >> 3) & 1) << 3);
    return (r & 1) | ((r >> 1) & 6) | ((((r >> 1) ^ (r >> 3)) & 1) << 3);
  }
  if (SW == SW_LOWREG) return ((r & 3) << 1) | ((r >> 2) & 1);
  return (r >> 1) & 7;  // NG = 8: two rows share the 256-byte bank window
}

// Element offset of (row r, column c) in a swizzled tile with NG granules per row.
template <int NG, int SW = SW_MIN>
__device__ __forceinline__ int soff(int r, int c) {
  return r * (NG * 8) + (((c >> 3) ^ swz<NG, SW>(r)) << 3) + (c & 7);
}

// 16-byte read of logical granule `gr` of row r.
template <int NG, int SW = SW_MIN>
__device__ __forceinline__ u32x4 lds_row16(const uint16_t* X, int r, int gr) {
  return *reinterpret_cast<const u32x4*>(X + r * (NG * 8) + ((gr ^ swz<NG, SW>(r)) << 3));
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// ds_read_b64_tr_b16: within each group of 16 lanes, lane i supplies the address of
// 4 consecutive 16-bit values (row i/4, columns 4*(i%4)..+3 of a 4x16 block) and
// receives column i of the block: the 4 values of rows 0..3.
__device__ __forceinline__ u32x2 lds_tr16(const uint16_t* p) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(u32x2, r);
}

// MFMA operand read transposed from a swizzled row-major tile X[k][n]: for column
// n = n0 + lane%16 the lane gets slots 0..3 = X[k0 + 0..3][n] and slots
// 4..7 = X[k1 + 0..3][n].
template <int NG, int SW = SW_MIN>
__device__ __forceinline__ u32x4 lds_tr_operand(const uint16_t* X, int k0, int k1, int n0) {
  const int i = threadIdx.x & 15;
  const int c = n0 + 4 * (i & 3);
  const u32x2 a = lds_tr16(X + soff<NG, SW>(k0 + (i >> 2), c));
  const u32x2 b = lds_tr16(X + soff<NG, SW>(k1 + (i >> 2), c));
  u32x4 r = {a[0], a[1], b[0], b[1]};
  return r;
}

// ---------------------------------------------------------------------------
// Workgroup order.  Grids are 1-D; the hardware hands consecutive workgroup ids to
// the 8 XCDs in turn.  map_block turns id L into (rank, head): heads are split
// into 8 equal sets, one per XCD, so all tiles of a head share one L2; within an
// XCD tiles go out rank 0 first.  Callers map rank 0 to the tile with the most
// work under the causal mask.
__device__ __forceinline__ void map_block(int L, int n_heads, int& rank, int& head) {
  if ((n_heads & 7) == 0) {
    const int x = L & 7, s = L >> 3, hpx = n_heads >> 3;
    rank = s / hpx;
    head = x * hpx + s % hpx;
  } else {
    rank = L / n_heads;
    head = L % n_heads;
  }
}

// ---------------------------------------------------------------------------
// Direct global -> LDS copies (global_load_lds_dwordx4 / _dword).  Every lane
// supplies its own global address; the data of lane L lands at lds_base + size*L,
// so one wave instruction fills 64*size contiguous LDS bytes.  lds_base must be
// wave-uniform (it goes through M0).  The copy is tracked by vmcnt only: the
// kernels wait for it explicitly (wait_vmem / wait_vmem_n) before the barrier
// that publishes it.
//
// The copies are issued as inline assembly.  Through the compiler builtin, every
// LDS read that the compiler cannot prove disjoint from an in-flight copy gets an
// s_waitcnt vmcnt(0) in front of it; with the LDS buffer chosen at run time that
// is every read, so each tile would wait for the copy of the tile two ahead that
// it has just started.  The kernels never read a buffer while a copy into it is in
// flight (the buffer being filled is the one consumed two iterations earlier).
// 32-bit LDS address of a wave-uniform LDS pointer, in a scalar register.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const void __attribute__((address_space(3)))*)p);
}
__device__ __forceinline__ void dma16(const void* gsrc, void* lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gsrc), "s"(lds_addr(lds_base))
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* gsrc, void* lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(gsrc), "s"(lds_addr(lds_base))
               : "memory", "m0");
}

// Copies through a buffer resource.  A raw resource (no stride, no swizzle) covers
// `bytes` bytes from `base`; a lane whose offset lies at or past the end reads
// zeros, and an LDS-destination load writes those zeros.  With the resource based
// at the first row of a tile and sized to the rows that exist, each lane's offset
// is the same for every tile, so the offsets stay in registers, a copy costs no
// vector ALU work and rows past the end arrive as zeros.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 buf_rsrc(const void* base, int bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));  // stride 0
  r[2] = __builtin_amdgcn_readfirstlane(bytes);
  r[3] = 0x00020000;  // 32-bit data format: plain byte addressing on gfx9-family parts
  return r;
}
// LDS byte address of a wave-uniform pointer into LDS (the low half of its
// generic address), in a scalar register.
__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(p));
}
// 16 bytes per lane from rsrc + voff into LDS at lds + OFF + 16 * lane.
template <int OFF>
__device__ __forceinline__ void bdma16(int voff, const i32x4& rsrc, uint32_t lds) {
  asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(lds), "n"(OFF)
               : "memory", "m0", "scc");
}
// 4 bytes per lane from rsrc + voff into LDS at lds + 4 * lane.
__device__ __forceinline__ void bdma4(int voff, const i32x4& rsrc, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(lds)
               : "memory", "m0");
}
// 16-bit stores through a buffer resource: the low (store16_lo) or high
// (store16_hi) half of `data` to rsrc + voff.  A lane whose offset lies at or past
// the resource's end stores nothing, so out-of-range elements need no branch.
__device__ __forceinline__ void bstore16_lo(uint32_t data, int voff, const i32x4& rsrc) {
  asm volatile("buffer_store_short %0, %1, %2, 0 offen" : : "v"(data), "v"(voff), "s"(rsrc) : "memory");
}
__device__ __forceinline__ void bstore16_hi(uint32_t data, int voff, const i32x4& rsrc) {
  asm volatile("buffer_store_short_d16_hi %0, %1, %2, 0 offen" : : "v"(data), "v"(voff), "s"(rsrc)
               : "memory");
}

// 8-byte store of `data` to rsrc + voff (voff a multiple of 8); a lane whose offset
// lies at or past the resource's end stores nothing.
__device__ __forceinline__ void bstore64(const u32x2& data, int voff, const i32x4& rsrc) {
  asm volatile("buffer_store_dwordx2 %0, %1, %2, 0 offen" : : "v"(data), "v"(voff), "s"(rsrc)
               : "memory");
}

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// s_waitcnt vmcnt(N): at most N vector-memory operations of this wave still
// outstanding.  Vector memory loads complete in issue order, so this waits for all
// but the N most recent.
template <int N>
__device__ __forceinline__ void wait_vmem_n() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Workgroup barrier for LDS tiles.  __syncthreads() carries a release fence that
// the compiler implements with vmcnt(0), which would also wait for direct copies
// still in flight for later tiles.  Here each wave first waits for exactly the
// copies it needs (wait_vmem / wait_vmem_n), then for its own LDS stores; the asm
// clobbers keep the compiler from moving memory accesses across, and the
// LDS-only acquire fence orders later LDS reads after the barrier.
// Workgroup barrier that leaves the wave's LDS reads in flight: for barriers whose
// purpose is ordering the direct-to-LDS copies of other buffers (the operand
// reads outstanding at the barrier are of the buffer being computed on).
__device__ __forceinline__ void tile_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  asm volatile("" ::: "memory");
}

// Fill a swizzled ROWS x (NG*8) tile from rows row0.. of a row-major matrix with
// NG*8 columns; rows at or past n_rows read row n_rows-1 instead (callers mask
// them).  NT threads; each wave issues ROWS*NG/NT copies of 1 KB.
template <int NG, int ROWS, int NT = 256, int SW = SW_MIN>
__device__ __forceinline__ void dma_tile(const uint16_t* __restrict__ g, int row0, int n_rows,
                                         uint16_t* lds, int w, int lane) {
  constexpr int PER_WAVE = ROWS * NG / NT;
  static_assert(PER_WAVE >= 1 && PER_WAVE * NT == ROWS * NG, "tile must split evenly over waves");
#pragma unroll
  for (int c = 0; c < PER_WAVE; ++c) {
    const int blk = PER_WAVE * w + c;
    const int ph = blk * 64 + lane;  // physical granule this lane fills
    const int r = ph / NG;
    const int j = (ph % NG) ^ swz<NG, SW>(r);
    const int rr = min(row0 + r, n_rows - 1);
    dma16(g + (size_t)rr * (NG * 8) + 8 * j, lds + blk * 64 * 8);
  }
}

// ---------------------------------------------------------------------------
// Padded LDS tiles (the kernels whose score products are 16x16x32 MFMAs).  A pair
// of ROWS-row tiles of the same shape (Q and dO, or K and V) is stored as 2*ROWS
// rows of D + 16 16-bit elements: the 32-byte pad per row spreads the rows over
// the banks.  Measured on an MI355X for the 16x16x32 operand patterns (16-byte
// reads of 16 consecutive rows, transposed reads of 4 rows x 32 bytes), the
// 288-byte (D = 128) and 160-byte (D = 64) strides run within a few percent of the
// best XOR swizzle, and every operand of a tile is then a fixed offset from one
// per-lane base address, which keeps address registers out of the inner loop.
template <int D>
struct PadTile {
  static constexpr int RS = D + 16;           // row stride in elements
  static constexpr int GR = RS / 8;           // 16-byte granules per row, pad included
  static constexpr int NG = D / 8;            // data granules per row
};

// 16-byte read of granule gr of row r.
template <int D>
__device__ __forceinline__ u32x4 pad_row16(const uint16_t* X, int r, int gr) {
  return *reinterpret_cast<const u32x4*>(X + r * PadTile<D>::RS + 8 * gr);
}

// Transposed MFMA operand (as lds_tr_operand) from a padded tile.
template <int D>
__device__ __forceinline__ u32x4 pad_tr_operand(const uint16_t* X, int k0, int k1, int n0) {
  const int i = threadIdx.x & 15;
  const int c = n0 + 4 * (i & 3);
  const u32x2 a = lds_tr16(X + (k0 + (i >> 2)) * PadTile<D>::RS + c);
  const u32x2 b = lds_tr16(X + (k1 + (i >> 2)) * PadTile<D>::RS + c);
  u32x4 r = {a[0], a[1], b[0], b[1]};
  return r;
}

// Fill a pair of padded ROWS-row tiles (tile 0 from g0, tile 1 from g1; matrices of
// D columns, rows row0..; rows at or past n_rows read row n_rows-1, callers mask
// them).  The pair is 2*ROWS*GR granules, copied by 4 waves in 1-KB instructions
// (PER_WAVE each); each wave's instructions fall in one tile.  Pad granules receive
// a copy of granule 0 of their row.  part(c, ...) issues instruction c of the
// calling wave, so the copy can be spread over a stream of other work.
template <int D, int ROWS>
struct PadPairCopy {
  using T = PadTile<D>;
  static constexpr int TILE_SLOTS = ROWS * T::GR;
  static constexpr int PER_WAVE = 2 * TILE_SLOTS / (4 * 64);
  static_assert(PER_WAVE * 4 * 64 == 2 * TILE_SLOTS && TILE_SLOTS % (2 * 64) == 0,
                "each wave must copy whole instructions within one tile");
  static __device__ __forceinline__ void part(int c, const uint16_t* __restrict__ g0,
                                              const uint16_t* __restrict__ g1, int row0, int n_rows,
                                              uint16_t* lds, int w, int lane) {
    const uint16_t* __restrict__ src = w < 2 ? g0 : g1;
    const int blk = PER_WAVE * w + c;
    const int slot = blk * 64 + lane - (w < 2 ? 0 : TILE_SLOTS);  // slot within its tile
    const int r = slot / T::GR, gr = slot % T::GR;
    const int rr = min(row0 + r, n_rows - 1);
    dma16(src + (size_t)rr * D + 8 * (gr < T::NG ? gr : 0), lds + blk * 64 * 8);
  }
};

// The same pair fill through buffer resources (one per source tile, based at the
// tile's first row): instruction c of wave w copies LDS bytes
// lds_wave_offset(w) + lds_offset<c> .. +1023 of the pair from byte
// src_offset(c, w, lane) of its tile, per lane.  Rows past the resource's end
// arrive as zeros.
template <int D, int ROWS>
struct PadPairDma {
  using T = PadTile<D>;
  static constexpr int TILE_SLOTS = ROWS * T::GR;
  static constexpr int PER_WAVE = 2 * TILE_SLOTS / (4 * 64);
  static_assert(PER_WAVE * 4 * 64 == 2 * TILE_SLOTS && TILE_SLOTS % (2 * 64) == 0,
                "each wave must copy whole instructions within one tile");
  static __device__ __forceinline__ int src_offset(int c, int w, int lane) {
    const int slot = (PER_WAVE * w + c) * 64 + lane - (w < 2 ? 0 : TILE_SLOTS);
    const int r = slot / T::GR, gr = slot % T::GR;
    return 2 * (r * D + 8 * (gr < T::NG ? gr : 0));
  }
  // (the wave index enters at run time, the instruction index as an immediate)
  static __device__ __forceinline__ uint32_t lds_wave_offset(int w) { return (uint32_t)(PER_WAVE * w * 1024); }
  template <int C>
  static constexpr int lds_offset = C * 1024;
};

// A ROWS x COLS block of a 16-bit matrix with a run-time row stride (elements; rows
// 16-byte aligned) copied to LDS as rows of COLS + 8 PADG elements (the PADG pad
// granules of a row receive a copy of its granule 0), in 1-KB wave instructions:
// instruction c of wave w fills LDS bytes lds_wave_offset(w) + lds_offset<c> ..
// +1023 from byte src_offset(c, w, lane, stride) of a buffer resource based at the
// block's first element.  Rows beyond the resource's end arrive as zeros.
template <int ROWS, int COLS, int PADG>
struct StridedTileDma {
  static constexpr int RS = COLS + 8 * PADG;  // LDS row stride, elements
  static constexpr int GR = COLS / 8 + PADG;  // 16-byte granules per LDS row
  static constexpr int PER_WAVE = ROWS * GR / 256;
  static_assert(PER_WAVE * 256 == ROWS * GR, "whole 1-KB instructions per wave");
  static __device__ __forceinline__ int src_offset(int c, int w, int lane, int stride) {
    const int slot = (PER_WAVE * w + c) * 64 + lane;
    const int r = slot / GR, g = slot % GR;
    return 2 * (r * stride + 8 * (g < COLS / 8 ? g : 0));
  }
  static __device__ __forceinline__ uint32_t lds_wave_offset(int w) { return (uint32_t)(PER_WAVE * w * 1024); }
  template <int C>
  static constexpr int lds_offset = C * 1024;
};

template <int D, int ROWS>
__device__ __forceinline__ void dma_pad_pair(const uint16_t* __restrict__ g0,
                                             const uint16_t* __restrict__ g1, int row0, int n_rows,
                                             uint16_t* lds, int w, int lane) {
#pragma unroll
  for (int c = 0; c < PadPairCopy<D, ROWS>::PER_WAVE; ++c)
    PadPairCopy<D, ROWS>::part(c, g0, g1, row0, n_rows, lds, w, lane);
}

// ---------------------------------------------------------------------------
// Instruction-scheduling hints (LLVM AMDGPU sched_group_barrier): ask the
// scheduler to place the next `n` instructions of a class here, in program order
// of the hints; sched_fence() keeps instructions from moving across it.
enum : int { SG_VALU = 0x002, SG_MFMA = 0x008, SG_VMEM = 0x010, SG_DSR = 0x100, SG_DSW = 0x200 };
#define sched_group(mask, n) __builtin_amdgcn_sched_group_barrier((mask), (n), 0)
#define sched_fence() __builtin_amdgcn_sched_barrier(0)

// Compile-time loop: f(std::integral_constant<int, 0>()), ..., f(..., N-1>()).
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>()), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>());
}

// Philox4x32-10, the counter-based generator of Salmon, Moraes, Dror and Shaw
// ("Parallel random numbers: as easy as 1, 2, 3", SC 2011): ten rounds, each
// (c0, c1, c2, c3) -> (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1,
// lo(M0 c0)), with the key bumped by the Weyl constants before every round but the
// first.  The dropout mask draws one call per 4 x 4 block of (query, key) positions.
__device__ __forceinline__ u32x4 philox4x32_10(u32x4 c, uint32_t k0, uint32_t k1) {
  constexpr uint32_t kM0 = 0xD2511F53u, kM1 = 0xCD9E8D57u;
  constexpr uint32_t kW0 = 0x9E3779B9u, kW1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += kW0;
      k1 += kW1;
    }
    const uint64_t p0 = (uint64_t)kM0 * c[0];
    const uint64_t p1 = (uint64_t)kM1 * c[2];
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    u32x4 n = {hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0};
    c = n;
  }
  return c;
}

// Keep factor of one element: its byte of the block's output below keep_t keeps
// it, with factor scale.
__device__ __forceinline__ float keep_factor(uint32_t word, int byte, uint32_t keep_t, float scale) {
  return ((word >> (8 * byte)) & 0xffu) < keep_t ? scale : 0.f;
}

// 4 x 4 transpose across the four lanes q = 0..3 of a quad: word w of lane q
// becomes what word q of lane w held.  Two exchange stages (lanes q ^ 2, then
// q ^ 1) through DPP quad permutations, each keeping or taking two words.
// Lets the four lanes that share a set of 4 x 4 dropout blocks each draw one
// block's Philox output and hand the others their parts of it.
__device__ __forceinline__ u32x4 quad_transpose(u32x4 m, int q) {
  auto x2 = [](uint32_t v) { return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false); };
  auto x1 = [](uint32_t v) { return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false); };
  const bool b1 = q & 2, b0 = q & 1;
  u32x4 p = {x2(m[2]), x2(m[3]), x2(m[0]), x2(m[1])};
  m = {b1 ? p[0] : m[0], b1 ? p[1] : m[1], b1 ? m[2] : p[2], b1 ? m[3] : p[3]};
  p = {x1(m[1]), x1(m[0]), x1(m[3]), x1(m[2])};
  return {b0 ? p[0] : m[0], b0 ? m[1] : p[1], b0 ? p[2] : m[2], b0 ? m[3] : p[3]};
}

// Whether no entry of slot table s comes before slot v: a value made in slot v
// (first in its slot) is ready for every item placed by s.
template <int A, int B>
constexpr bool none_before(const int (&s)[A][B], int v) {
  for (int a = 0; a < A; ++a)
    for (int b = 0; b < B; ++b)
      if (s[a][b] < v) return false;
  return true;
}

// Byte transpose within a lane: byte r of word c of the result is byte c of word r
// of x (eight byte permutations).
__device__ __forceinline__ u32x4 byte_transpose(const u32x4& x) {
  const uint32_t u01 = __builtin_amdgcn_perm(x[1], x[0], 0x05010400u);  // bytes 0-1 of x0, x1
  const uint32_t u23 = __builtin_amdgcn_perm(x[3], x[2], 0x05010400u);
  const uint32_t v01 = __builtin_amdgcn_perm(x[1], x[0], 0x07030602u);  // bytes 2-3
  const uint32_t v23 = __builtin_amdgcn_perm(x[3], x[2], 0x07030602u);
  return {__builtin_amdgcn_perm(u23, u01, 0x05040100u), __builtin_amdgcn_perm(u23, u01, 0x07060302u),
          __builtin_amdgcn_perm(v23, v01, 0x05040100u), __builtin_amdgcn_perm(v23, v01, 0x07060302u)};
}

// max(a, b, c) in one v_max3_f32.  fmaxf on MFMA results costs a canonicalizing
// v_max_f32 per input as well (the IEEE mode quiets signalling NaNs first); the
// scores here are finite or -inf.
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Makes a value opaque to the compiler (ON): it is computed once, where placed,
// and not rematerialized next to its use (a repack right before the MFMA that
// reads it would be a VALU write of an MFMA source without wait states).
template <bool ON>
__device__ __forceinline__ void pin(u32x2& v) {
  if constexpr (ON) asm volatile("" : "+v"(v));
}

// Element i (0..3) of four 16-bit values packed in a u32x2, as float.
template <int DT>
__device__ __forceinline__ float elem4(const u32x2& w, int i) {
  return (i & 1) ? Dt<DT>::hi(w[i >> 1]) : Dt<DT>::lo(w[i >> 1]);
}

// 16-byte global load/store helpers.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

__device__ __forceinline__ u32x4 zero_u4() {
  u32x4 z = {0u, 0u, 0u, 0u};
  return z;
}

}  // namespace fa
