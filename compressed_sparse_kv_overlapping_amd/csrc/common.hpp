// Device-side helpers shared by the gfx950 kernels: storage dtypes, bf16
// rounding, wave shuffles and MFMA fragment wrappers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cskv {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int v8i32_t __attribute__((ext_vector_type(8)));
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
// fp32 -> bf16, round to nearest even (the gfx950 packed conversion)
typedef __bf16 hw_bf16x2_t __attribute__((ext_vector_type(2)));
typedef float hw_f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(hw_f32x2_t{lo, hi}, hw_bf16x2_t));
}
__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return pack_bf16x2(f, 0.f) & 0xffffu; }

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

// 8 consecutive elements kept in their storage format (16 bytes of bf16 or
// 32 bytes of fp32) and widened on use.
template <class T> struct Raw8;
template <> struct Raw8<bf16_t> {
  uint4 v;
  __device__ __forceinline__ void load(const bf16_t* p) { v = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void load_nt(const bf16_t* p) {
    const u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    v = make_uint4(a.x, a.y, a.z, a.w);
  }
  __device__ __forceinline__ float operator[](int i) const {
    const uint32_t w = i < 2 ? v.x : i < 4 ? v.y : i < 6 ? v.z : v.w;
    return (i & 1) ? bf16_hi(w) : bf16_lo(w);
  }
};
template <> struct Raw8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = reinterpret_cast<const float4*>(p)[0];
    b = reinterpret_cast<const float4*>(p)[1];
  }
  __device__ __forceinline__ void load_nt(const float* p) {
    const u32x4 u = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p) + 1);
    a = make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w));
    b = make_float4(__uint_as_float(w.x), __uint_as_float(w.y), __uint_as_float(w.z), __uint_as_float(w.w));
  }
  __device__ __forceinline__ float operator[](int i) const {
    return i == 0 ? a.x : i == 1 ? a.y : i == 2 ? a.z : i == 3 ? a.w
         : i == 4 ? b.x : i == 5 ? b.y : i == 6 ? b.z : b.w;
  }
};

// 4 consecutive elements in storage format (8 bytes bf16, 16 bytes fp32).
template <class T> struct Raw4;
template <> struct Raw4<bf16_t> {
  uint2 v;
  __device__ __forceinline__ void load(const bf16_t* p) { v = *reinterpret_cast<const uint2*>(p); }
  __device__ __forceinline__ void load_nt(const bf16_t* p) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 a = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    v = make_uint2(a.x, a.y);
  }
  __device__ __forceinline__ float operator[](int i) const {
    const uint32_t w = i < 2 ? v.x : v.y;
    return (i & 1) ? bf16_hi(w) : bf16_lo(w);
  }
};
template <> struct Raw4<float> {
  float4 a;
  __device__ __forceinline__ void load(const float* p) { a = *reinterpret_cast<const float4*>(p); }
  __device__ __forceinline__ void load_nt(const float* p) {
    const u32x4 u = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    a = make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w));
  }
  __device__ __forceinline__ float operator[](int i) const {
    return i == 0 ? a.x : i == 1 ? a.y : i == 2 ? a.z : a.w;
  }
};
// 2 consecutive elements in storage format (4 bytes bf16, 8 bytes fp32).
template <class T> struct Raw2;
template <> struct Raw2<bf16_t> {
  uint32_t v;
  __device__ __forceinline__ void load(const bf16_t* p) { v = *reinterpret_cast<const uint32_t*>(p); }
  __device__ __forceinline__ void load_nt(const bf16_t* p) {
    v = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
  }
  __device__ __forceinline__ float operator[](int i) const { return i ? bf16_hi(v) : bf16_lo(v); }
};
template <> struct Raw2<float> {
  float a, b;
  __device__ __forceinline__ void load(const float* p) { a = p[0]; b = p[1]; }
  __device__ __forceinline__ void load_nt(const float* p) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 u = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    a = __uint_as_float(u.x);
    b = __uint_as_float(u.y);
  }
  __device__ __forceinline__ float operator[](int i) const { return i ? b : a; }
};

template <class T, int N> struct RawN;
template <class T> struct RawN<T, 2> : Raw2<T> {};
template <class T> struct RawN<T, 8> : Raw8<T> {};
template <class T> struct RawN<T, 4> : Raw4<T> {};

// N consecutive fp32 stored as the output dtype.
template <class T, int N> struct StoreN;
template <class T> struct StoreN<T, 8> {
  static __device__ __forceinline__ void store(T* p, const float* v) { Row8<T>::store(p, v); }
};
template <> struct StoreN<bf16_t, 4> {
  static __device__ __forceinline__ void store(bf16_t* p, const float* v) {
    *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
  }
};
template <> struct StoreN<float, 4> {
  static __device__ __forceinline__ void store(float* p, const float* v) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
};

// Raw buffer stores: the hardware drops stores whose offset is at or past
// num_records, so a store can be issued unconditionally and masked by its
// offset (keeps loops free of conditional memory operations).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
template <class T, int N> struct BufStoreN;
template <> struct BufStoreN<bf16_t, 2> {
  static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, uint32_t off, const float* v) {
    __builtin_amdgcn_raw_buffer_store_b32(pack_bf16x2(v[0], v[1]), r, off, 0, 0);
  }
};
template <> struct BufStoreN<float, 2> {
  static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, uint32_t off, const float* v) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 w = {__float_as_uint(v[0]), __float_as_uint(v[1])};
    __builtin_amdgcn_raw_buffer_store_b64(w, r, off, 0, 0);
  }
};
template <> struct BufStoreN<bf16_t, 4> {
  static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, uint32_t off, const float* v) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    u32x2 w = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    __builtin_amdgcn_raw_buffer_store_b64(w, r, off, 0, 0);
  }
};
template <> struct BufStoreN<bf16_t, 8> {
  static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, uint32_t off, const float* v) {
    u32x4 w = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
               pack_bf16x2(v[6], v[7])};
    __builtin_amdgcn_raw_buffer_store_b128(w, r, off, 0, 0);
  }
};
template <> struct BufStoreN<float, 4> {
  static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, uint32_t off, const float* v) {
    u32x4 w = {__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
    __builtin_amdgcn_raw_buffer_store_b128(w, r, off, 0, 0);
  }
};
template <> struct BufStoreN<float, 8> {
  static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, uint32_t off, const float* v) {
    BufStoreN<float, 4>::store(r, off, v);
    BufStoreN<float, 4>::store(r, off + 16, v + 4);
  }
};

// ---------------------------------------------------------------- shuffles
__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }

// Combine a value with the one held by lane ^ 16 (or ^ 32) through the gfx950
// lane-half swaps (plain VALU, no LDS round trip).  Both lanes of a pair see
// the two values in the same order, so they get bitwise equal results.
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

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

// ------------------------------------------------------------ LDS copies
// One 16-byte copy per lane from global memory straight into LDS: lane i's
// bytes land at lds_base + 16 i (lds_base wave-uniform).  Issued through
// inline asm so that the compiler adds no waits of its own before LDS reads:
// a buffer filled this way is read only after an explicit
// "s_waitcnt vmcnt(0)" and a barrier.  No memory clobber, so other loads may
// move across it.
__device__ __forceinline__ unsigned lds_offset(const void* p) {
  return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}
__device__ __forceinline__ void dma16(const char* src, unsigned lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(src), "s"(lds_base) : "m0");
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
