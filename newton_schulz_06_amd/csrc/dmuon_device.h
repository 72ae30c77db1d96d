// Device helpers shared by libdmuon's kernel files: vector types, fp32 <->
// bf16 conversion, explicit global-memory accessors, a fixed-order
// wavefront sum and the task lookup of grouped launches.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace dmuon {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest even, NaN stays NaN: gfx950 converts in
// hardware (v_cvt_pk_bf16_f32), without a branch.
__device__ __forceinline__ uint16_t to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ uint32_t to_bf16x2(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ float from_bf16(uint16_t h) {
  return __uint_as_float((uint32_t)h << 16);
}

// Global-memory accessors.  Device pointers reach the kernels through task
// tables, where the compiler cannot prove their address space; without an
// explicit global (address space 1) access it emits flat instructions,
// which also wait on the LDS counter.
#define GMEM __attribute__((address_space(1)))
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float ld_f32(const float* p) { return *(const GMEM float*)p; }
__device__ __forceinline__ void st_f32(float* p, float v) { *(GMEM float*)p = v; }
__device__ __forceinline__ f32x4 ld_f32x4(const float* p) { return *(const GMEM f32x4*)p; }
__device__ __forceinline__ void st_f32x4(float* p, f32x4 v) { *(GMEM f32x4*)p = v; }
__device__ __forceinline__ uint16_t ld_u16(const uint16_t* p) { return *(const GMEM uint16_t*)p; }
__device__ __forceinline__ void st_u16(uint16_t* p, uint16_t v) { *(GMEM uint16_t*)p = v; }
__device__ __forceinline__ u32x2 ld_u32x2(const uint16_t* p) { return *(const GMEM u32x2*)p; }
__device__ __forceinline__ void st_u32x2(uint16_t* p, u32x2 v) { *(GMEM u32x2*)p = v; }
__device__ __forceinline__ void st_u32x4(uint16_t* p, u32x4 v) { *(GMEM u32x4*)p = v; }
__device__ __forceinline__ uint4 ld_u128(const void* p) {
  const u32x4 w = *(const GMEM u32x4*)p;
  return make_uint4(w.x, w.y, w.z, w.w);
}

// Streaming accessors for data touched once per kernel (gradients, momentum
// buffers, optimizer state): nontemporal loads and stores keep them from
// displacing cached lines.  Measured on MI355X: AdamW 5.44 -> 5.99 TB/s,
// the clipping norm pass 9% faster.  Results that another kernel reads
// soon after keep ordinary stores: nontemporal ones slowed the SYRK, whose
// output the polynomial reads next, by 9%.  The fp32 master X and bf16 X of
// matrices on 256-wide tiles (p >= 1024: gigabytes per batch, far beyond
// the caches before their next use) are streamed too: Llama-8B X update
// 41.3 -> 40.5 ms per step.
__device__ __forceinline__ f32x4 ld_f32x4_nt(const float* p) {
  return __builtin_nontemporal_load((const GMEM f32x4*)p);
}
__device__ __forceinline__ void st_f32x4_nt(float* p, f32x4 v) {
  __builtin_nontemporal_store(v, (GMEM f32x4*)p);
}
__device__ __forceinline__ float ld_f32_nt(const float* p) {
  return __builtin_nontemporal_load((const GMEM float*)p);
}
__device__ __forceinline__ void st_f32_nt(float* p, float v) {
  __builtin_nontemporal_store(v, (GMEM float*)p);
}
__device__ __forceinline__ void st_u16_nt(uint16_t* p, uint16_t v) {
  __builtin_nontemporal_store(v, (GMEM uint16_t*)p);
}
__device__ __forceinline__ u32x2 ld_u32x2_nt(const uint16_t* p) {
  return __builtin_nontemporal_load((const GMEM u32x2*)p);
}
__device__ __forceinline__ void st_u32x2_nt(uint16_t* p, u32x2 v) {
  __builtin_nontemporal_store(v, (GMEM u32x2*)p);
}

__device__ __forceinline__ float load1(const void* base, int dtype, size_t i) {
  return dtype == 0 ? ld_f32(static_cast<const float*>(base) + i)
                    : from_bf16(ld_u16(static_cast<const uint16_t*>(base) + i));
}

__device__ __forceinline__ f32x4 load4(const void* base, int dtype, size_t i) {
  f32x4 r;
  if (dtype == 0) {
    r = ld_f32x4_nt(static_cast<const float*>(base) + i);
  } else {
    const u32x2 w = ld_u32x2_nt(static_cast<const uint16_t*>(base) + i);
    r[0] = __uint_as_float(w.x << 16);
    r[1] = __uint_as_float(w.x & 0xffff0000u);
    r[2] = __uint_as_float(w.y << 16);
    r[3] = __uint_as_float(w.y & 0xffff0000u);
  }
  return r;
}

__device__ __forceinline__ u32x2 pack_bf16x4(float a, float b, float c, float d) {
  u32x2 w;
  w.x = to_bf16x2(a, b);
  w.y = to_bf16x2(c, d);
  return w;
}

__device__ __forceinline__ f32x4 unpack_bf16x4(u32x2 w) {
  f32x4 r;
  r[0] = __uint_as_float(w.x << 16);
  r[1] = __uint_as_float(w.x & 0xffff0000u);
  r[2] = __uint_as_float(w.y << 16);
  r[3] = __uint_as_float(w.y & 0xffff0000u);
  return r;
}

// 16-bit operand formats of the bf16-path NS products: Op16<0> bf16,
// Op16<1> fp16 (IEEE half: 5 exponent bits, 10 fraction bits).  Both
// convert fp32 with round to nearest even and feed the same-rate gfx950
// MFMA (v_mfma_f32_32x32x16_bf16 / _f16).  A hi/lo master X keeps its
// remainder scaled by kLoScale: x - hi is at most half an fp16 spacing of
// x, which falls in fp16's subnormal range for |x| below 2^-3; scaled by
// 2^11 it stays normal down to |x| = 2^-14 (bf16's exponent range needs no
// scale).
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

template <int H>
struct Op16;

// kAScale / kBScale: the A and B operands are stored times these powers of
// two and their products divided by them in the consumers' epilogues (exact
// either way).  With ||X|| near 1, the off-diagonal entries of A = X X^T
// and A^2 fall below fp16's normal range (2^-14) as p grows; scaled they stay
// normal, with room up to |A| = 16 and |B| = 64 (the NS iterates keep
// |A| <= ~1.5 and |B| <= ~12 with the quintic).
template <>
struct Op16<0> {
  using vec8 = bf16x8;
  static constexpr float kLoScale = 1.f;
  static constexpr float kAScale = 1.f;
  static constexpr float kBScale = 1.f;
  static __device__ __forceinline__ uint16_t to(float f) { return to_bf16(f); }
  static __device__ __forceinline__ uint32_t to2(float a, float b) { return to_bf16x2(a, b); }
  static __device__ __forceinline__ float from(uint16_t h) { return from_bf16(h); }
  // element 0 (low half) and element 1 (high half) of a packed pair
  static __device__ __forceinline__ float e0(uint32_t w) { return __uint_as_float(w << 16); }
  static __device__ __forceinline__ float e1(uint32_t w) {
    return __uint_as_float(w & 0xffff0000u);
  }
  static __device__ __forceinline__ f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Op16<1> {
  using vec8 = f16x8;
  static constexpr float kLoScale = 2048.f;
  static constexpr float kAScale = 4096.f;
  static constexpr float kBScale = 1024.f;
  static __device__ __forceinline__ uint16_t to(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);
  }
  static __device__ __forceinline__ uint32_t to2(float a, float b) {
    const f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  }
  static __device__ __forceinline__ float from(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
  }
  static __device__ __forceinline__ float e0(uint32_t w) { return from((uint16_t)(w & 0xffffu)); }
  static __device__ __forceinline__ float e1(uint32_t w) { return from((uint16_t)(w >> 16)); }
  static __device__ __forceinline__ f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

template <int H>
__device__ __forceinline__ u32x2 pack4(float a, float b, float c, float d) {
  u32x2 w;
  w.x = Op16<H>::to2(a, b);
  w.y = Op16<H>::to2(c, d);
  return w;
}

template <int H>
__device__ __forceinline__ f32x4 unpack4(u32x2 w) {
  f32x4 r;
  r[0] = Op16<H>::e0(w.x);
  r[1] = Op16<H>::e1(w.x);
  r[2] = Op16<H>::e0(w.y);
  r[3] = Op16<H>::e1(w.y);
  return r;
}

// Last task whose tile_begin <= tile (tasks are sorted by tile_begin).
template <class Task>
__device__ __forceinline__ int find_task(const Task* tasks, int ntasks, int tile) {
  int lo = 0, hi = ntasks - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tasks[mid].tile_begin <= tile) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// --------------------------------------------------------------------------
// Wavefront sum: DPP within each row of 16 lanes, then cross-row shuffles.
// Every lane ends with the same value, summed in a fixed order.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, true));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_mov<0x141>(v);  // row_half_mirror
  v += dpp_mov<0x140>(v);  // row_mirror
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

}  // namespace
}  // namespace dmuon
