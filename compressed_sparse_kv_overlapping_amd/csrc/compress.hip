// Streaming KV compressor for gfx950.
//
// Method: "DeepSeek V4 comprimeix el context: aixi funcionen CSA i HCA",
// sections "DeepSeek comprimeix la dimensio temporal" and "Finestres
// solapades per evitar fronteres artificials": every entry is a weighted sum
// of the 512-dim shared-KV rows of an overlapping window, with a softmax over
// the window's tokens taken separately for every dimension.  Window of entry
// i: tokens [(i-1)m, (i+1)m) (2m tokens, stride m); tokens before 0 are left
// out of the softmax; logit of the token at window position p is z + b[p].
//
// Mapping: one wavefront per entry; each lane owns 8 consecutive dims, so a
// wave reads whole 512-wide rows (1 KiB in bf16) with 16-byte loads.  The
// window is walked in chunks of 8 tokens with an online per-dimension
// softmax (running max, rescaled sum and weighted sum held in registers, all
// in the exp2 domain).  Adjacent waves of a block handle adjacent entries, so
// the half window two entries share is read from HBM once and from L1/L2 the
// second time.  Blocks are mapped so that consecutive entry ranges stay on
// one XCD and share its L2.
#include "common.hpp"
#include "kernels.hpp"

namespace cskv {

constexpr int kD = 512;
constexpr int kCompressWaves = 4;
constexpr int kChunk = 8;

// Block id -> logical range index such that the ranges handled by one XCD
// are contiguous (the dispatcher deals block ids round-robin over 8 XCDs).
__device__ __forceinline__ int xcd_contiguous(int id, int G) {
  int q = G / 8, rem = G % 8;
  int x = id % 8, slot = id / 8;
  return x * q + (x < rem ? x : rem) + slot;
}

template <class T>
__global__ __launch_bounds__(64 * kCompressWaves) void compress_kernel(
    const T* __restrict__ x, const T* __restrict__ z, const float* __restrict__ bias, int m,
    int64_t e_begin, int64_t e_end, int entries_per_wave, T* __restrict__ out, int64_t ld_out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int d0 = lane * 8;
  const int blk = xcd_contiguous(blockIdx.x, gridDim.x);
  const float L2E = 1.4426950408889634f;
  for (int r = 0; r < entries_per_wave; ++r) {
    const int64_t e = e_begin + ((int64_t)blk * entries_per_wave + r) * kCompressWaves + wave;
    if (e >= e_end) return;
    const int p_lo = (e == 0) ? m : 0;            // tokens before 0 are absent
    const int64_t j0 = (e - 1) * (int64_t)m;      // token at window position 0
    float M[8], S[8], A[8];
#pragma unroll
    for (int d = 0; d < 8; ++d) { M[d] = -INFINITY; S[d] = 0.f; A[d] = 0.f; }
    for (int p0 = p_lo; p0 < 2 * m; p0 += kChunk) {
      const int nt = min(kChunk, 2 * m - p0);
      float lz[kChunk][8], xv[kChunk][8];
#pragma unroll
      for (int t = 0; t < kChunk; ++t) {
        if (t < nt) {
          const int64_t j = j0 + p0 + t;
          float bv[8];
          Row8<T>::load(z + j * kD + d0, lz[t]);
          Row8<T>::load(x + j * kD + d0, xv[t]);
          Row8<float>::load(bias + (int64_t)(p0 + t) * kD + d0, bv);
#pragma unroll
          for (int d = 0; d < 8; ++d) lz[t][d] = (lz[t][d] + bv[d]) * L2E;
        }
      }
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        float cm = lz[0][d];
#pragma unroll
        for (int t = 1; t < kChunk; ++t)
          if (t < nt) cm = fmaxf(cm, lz[t][d]);
        const float mn = fmaxf(M[d], cm);
        const float alpha = __builtin_amdgcn_exp2f(M[d] - mn);    // 0 on the first chunk (M = -inf)
        float s = 0.f, a = 0.f;
#pragma unroll
        for (int t = 0; t < kChunk; ++t) {
          if (t < nt) {
            const float w = __builtin_amdgcn_exp2f(lz[t][d] - mn);
            s += w;
            a = fmaf(w, xv[t][d], a);
          }
        }
        S[d] = fmaf(S[d], alpha, s);
        A[d] = fmaf(A[d], alpha, a);
        M[d] = mn;
      }
    }
    float o[8];
#pragma unroll
    for (int d = 0; d < 8; ++d) o[d] = A[d] / S[d];
    Row8<T>::store(out + e * ld_out + d0, o);
  }
}

template <class T>
static hipError_t launch_compress_t(const void* x, const void* z, const float* bias, int m,
                                    int64_t e_begin, int64_t e_end, void* out, int64_t ld_out,
                                    hipStream_t stream) {
  const int64_t n = e_end - e_begin;
  if (n <= 0) return hipSuccess;
  // enough blocks to fill 256 CUs several times; up to 16 entries per wave
  int64_t epw = n / (kCompressWaves * 2048);
  epw = epw < 1 ? 1 : (epw > 16 ? 16 : epw);
  const int64_t per_block = epw * kCompressWaves;
  const int64_t grid = (n + per_block - 1) / per_block;
  hipLaunchKernelGGL(compress_kernel<T>, dim3((unsigned)grid), dim3(64 * kCompressWaves), 0,
                     stream, (const T*)x, (const T*)z, bias, m, e_begin, e_end, (int)epw, (T*)out,
                     ld_out);
  return hipGetLastError();
}

hipError_t launch_compress(int dt, const void* x, const void* z, const float* bias, int m,
                           int64_t e_begin, int64_t e_end, void* out, int64_t ld_out,
                           hipStream_t stream) {
  if (dt == 0) return launch_compress_t<float>(x, z, bias, m, e_begin, e_end, out, ld_out, stream);
  return launch_compress_t<bf16_t>(x, z, bias, m, e_begin, e_end, out, ld_out, stream);
}

}  // namespace cskv
