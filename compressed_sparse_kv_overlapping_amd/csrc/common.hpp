// Device-side helpers shared by the gfx950 kernels: storage dtypes, bf16
// rounding, wave shuffles and MFMA fragment wrappers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cskv {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- dtypes
// Storage types: float (fp32), bf16 (raw uint16 bits), fp8 e4m3 (raw uint8,
// OCP format as consumed by the gfx950 fp8 MFMA).
struct bf16_t { uint16_t u; };
struct e4m3_t { uint8_t u; };

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// Load 8 consecutive elements starting at p (16-byte aligned for bf16, 32 for
// fp32) and widen them to fp32.
template <class T> struct Row8;
template <> struct Row8<float> {
  static __device__ __forceinline__ void load(const float* p, float v[8]) {
    float4 a = *reinterpret_cast<const float4*>(p);
    float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  static __device__ __forceinline__ void load_nt(const float* p, float v[8]) {
    const f32x4* q = reinterpret_cast<const f32x4*>(p);
    f32x4 a = __builtin_nontemporal_load(q);
    f32x4 b = __builtin_nontemporal_load(q + 1);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  static __device__ __forceinline__ void store(float* p, const float v[8]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
};
template <> struct Row8<bf16_t> {
  static __device__ __forceinline__ void widen(uint4 a, float v[8]) {
    v[0] = bf16_lo(a.x); v[1] = bf16_hi(a.x); v[2] = bf16_lo(a.y); v[3] = bf16_hi(a.y);
    v[4] = bf16_lo(a.z); v[5] = bf16_hi(a.z); v[6] = bf16_lo(a.w); v[7] = bf16_hi(a.w);
  }
  static __device__ __forceinline__ void load(const bf16_t* p, float v[8]) {
    widen(*reinterpret_cast<const uint4*>(p), v);
  }
  static __device__ __forceinline__ void load_nt(const bf16_t* p, float v[8]) {
    u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    widen(make_uint4(a.x, a.y, a.z, a.w), v);
  }
  static __device__ __forceinline__ void store(bf16_t* p, const float v[8]) {
    uint4 o;
    o.x = pack_bf16x2(v[0], v[1]); o.y = pack_bf16x2(v[2], v[3]);
    o.z = pack_bf16x2(v[4], v[5]); o.w = pack_bf16x2(v[6], v[7]);
    *reinterpret_cast<uint4*>(p) = o;
  }
};

// ---------------------------------------------------------------- shuffles
__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }

// Order-preserving map of an fp32 score to uint32 (larger score -> larger key);
// -0 is folded onto +0 so equal values get equal keys.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s + 0.0f);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k ^ 0x80000000u) : ~k;
  return __uint_as_float(u);
}

// ---------------------------------------------------------------- MFMA
// A fragment is 8 "k-slots" per lane.  For an MxN MFMA tile (M = N = MN) the
// lane l supplies row (A) / column (B) l % MN and the k-slots of lane group
// g = l / MN.  The hardware pairs slot t of lane group g in A with the same
// slot of the same group in B, so any consistent assignment of k values to
// (g, t) gives the full contraction; the kernels use that freedom to match
// the accumulator layout of one product to the operand layout of the next.
template <class T> struct Frag;
template <> struct Frag<bf16_t> { u32x4 v; };          // 8 bf16
template <> struct Frag<float> { float v[8]; };        // 8 fp32
template <> struct Frag<e4m3_t> { uint64_t v; };       // 8 fp8

template <class T> __device__ __forceinline__ void frag_load(Frag<T>& f, const T* p);
template <> __device__ __forceinline__ void frag_load<bf16_t>(Frag<bf16_t>& f, const bf16_t* p) {
  uint4 a = *reinterpret_cast<const uint4*>(p);
  f.v = u32x4{a.x, a.y, a.z, a.w};
}
template <> __device__ __forceinline__ void frag_load<float>(Frag<float>& f, const float* p) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
  f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}
template <> __device__ __forceinline__ void frag_load<e4m3_t>(Frag<e4m3_t>& f, const e4m3_t* p) {
  f.v = *reinterpret_cast<const uint64_t*>(p);
}

// 16x16 tile, 32 k per step (8 slots x 4 lane groups).
__device__ __forceinline__ void mma16(f32x4& c, const Frag<bf16_t>& a, const Frag<bf16_t>& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a.v),
                                              __builtin_bit_cast(bf16x8, b.v), c, 0, 0, 0);
}
__device__ __forceinline__ void mma16(f32x4& c, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int t = 0; t < 8; ++t) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[t], b.v[t], c, 0, 0, 0);
}
__device__ __forceinline__ void mma16(f32x4& c, const Frag<e4m3_t>& a, const Frag<e4m3_t>& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8((long)a.v, (long)b.v, c, 0, 0, 0);
}

// 32x32 tile, 16 k per step (8 slots x 2 lane groups).
__device__ __forceinline__ void mma32(f32x16& c, const Frag<bf16_t>& a, const Frag<bf16_t>& b) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a.v),
                                              __builtin_bit_cast(bf16x8, b.v), c, 0, 0, 0);
}
__device__ __forceinline__ void mma32(f32x16& c, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int t = 0; t < 8; ++t) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.v[t], b.v[t], c, 0, 0, 0);
}

}  // namespace cskv
