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
// Kernels: compress_small_kernel (m <= 4, the CSA scale) and
// compress_large_kernel (m > 4, the HCA scale) stream one scale each;
// compress_fused_kernel streams the raw rows once for both scales (with
// compress_join_kernel after it).  Every
// wave streams a contiguous range of entries and reads each raw row once;
// adjacent ranges hand over the half window they share.  Blocks are mapped
// so that consecutive ranges stay on one XCD and share its L2.
#include "common.hpp"
#include "kernels.hpp"
#include <cmath>

namespace cskv {

constexpr int kD = 512;

// Block id -> logical range index such that the ranges handled by one XCD
// are contiguous (the dispatcher deals block ids round-robin over 8 XCDs).
__device__ __forceinline__ int xcd_contiguous(int id, int G) {
  int q = G / 8, rem = G % 8;
  int x = id % 8, slot = id / 8;
  return x * q + (x < rem ? x : rem) + slot;
}

// ---------------------------------------------------------------------------
// Streaming compressor for small blocks (m <= 4), the CSA scale.
//
// A wave streams a contiguous range of entries and reads every token once.
// Block b (tokens [bm, bm+m)) feeds two windows: the second half of entry b
// (window positions m..2m-1) and the first half of entry b+1 (positions
// 0..m-1).  With the block maximum r of z (per dimension), a token's weight
// in either window factors as
//     exp(z + b_p - M) = 2^(z*log2e - r) * 2^((b_p - bmax)*log2e) * const,
// so each element needs one exp2, shared by both windows, times a
// per-position factor beta_p <= 1 precomputed once per block of waves (in
// LDS).  The two halves of an entry carry the references of their blocks
// and are joined with one exp2 per dimension, so the result equals the
// exact softmax up to rounding for any logit range.
constexpr float kBand = 8.f;
constexpr float kDown = 100.f;

// Next reference (log2 units) given a chunk/block maximum cm: raised to cm
// when cm > r + kBand (keeps weights <= 2^kBand); lowered when cm < r - kBand,
// but by at most kDown so that rescaled running sums (<= 2m * 2^kBand) stay
// finite.  Adjacent windows whose logits differ by more than ~kDown + 126
// log2 units would lose the smaller one to underflow.
__device__ __forceinline__ float next_ref(float r, float cm, bool have) {
  if (!have || cm > r + kBand) return cm;
  if (cm < r - kBand) return fmaxf(cm, r - kDown);
  return r;
}
#ifndef CSKV_SMALL_DPL
#define CSKV_SMALL_DPL 4
#endif
#ifndef CSKV_SMALL_RANGES
#define CSKV_SMALL_RANGES 8192
#endif
#ifndef CSKV_SMALL_RING
#define CSKV_SMALL_RING 3
#endif
constexpr int kSmallDpl = CSKV_SMALL_DPL;         // dims per lane
constexpr int kSmallRing = CSKV_SMALL_RING;       // register ring depth (blocks)
constexpr int64_t kSmallRanges = CSKV_SMALL_RANGES; // target number of entry ranges

template <class T, int M, int DPL>
__global__ __launch_bounds__(256) void compress_small_kernel(
    const T* __restrict__ x, const T* __restrict__ z, const float* __restrict__ bias,
    int64_t e_begin, int64_t e_end, int entries_per_wave, T* __restrict__ out, int64_t ld_out) {
  // DPL dims per lane; a wave covers 64*DPL dims, so kSlices waves share an
  // entry range (one per dim slice)
  constexpr int kSlices = kD / (64 * DPL);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int blk = xcd_contiguous(blockIdx.x, gridDim.x);
  const int gw = blk * 4 + wave;
  const int d0 = (gw % kSlices) * 64 * DPL + lane * DPL;
  const int64_t e0 = e_begin + (int64_t)(gw / kSlices) * entries_per_wave;
  const int64_t e1 = e0 + entries_per_wave < e_end ? e0 + entries_per_wave : e_end;
  const float L2E = 1.4426950408889634f;
  // output rows of this wave as a bounded buffer
  const __amdgpu_buffer_rsrc_t orsrc =
      make_rsrc(out + (e0 < e1 ? e0 : 0) * ld_out,
                e0 < e1 ? (uint32_t)((e1 - e0) * ld_out * sizeof(T)) : 0u);
  // beta_p = 2^((b_p - max_p b_p) * log2e) for positions 0..2M-1, in LDS
  __shared__ __attribute__((aligned(16))) float beta[2 * M][kD];
  for (int d = threadIdx.x; d < kD; d += 256) {
    float bm = bias[d];
    for (int p = 1; p < 2 * M; ++p) bm = fmaxf(bm, bias[(int64_t)p * kD + d]);
    for (int p = 0; p < 2 * M; ++p)
      beta[p][d] = __builtin_amdgcn_exp2f((bias[(int64_t)p * kD + d] - bm) * L2E);
  }
  __syncthreads();
  if (e0 >= e1) return;
  // carried first half (for the next entry) and its reference
  float cS[DPL], cA[DPL], cr[DPL];
#pragma unroll
  for (int d = 0; d < DPL; ++d) { cS[d] = 0.f; cA[d] = 0.f; cr[d] = 0.f; }
  int64_t bk = e0 > 0 ? e0 - 1 : 0;
  // ring of kRing register buffers (storage format): blocks are loaded
  // kRing - 1 blocks ahead of the one being folded
  constexpr int kRing = kSmallRing;
  RawN<T, DPL> zb[kRing][M], xb[kRing][M];
  // Loads are issued unconditionally (past the range they re-read the last
  // block) so the code stays straight-line and the wait counters only ever
  // wait for the block being folded, never for the prefetched ones.
  auto load_block = [&](int64_t b, RawN<T, DPL>* zz, RawN<T, DPL>* xx) {
    if (b > e1 - 1) b = e1 - 1;
#pragma unroll
    for (int t = 0; t < M; ++t) {
      const int64_t j = b * M + t;
      zz[t].load(z + j * kD + d0);
      xx[t].load(x + j * kD + d0);
    }
  };
  auto fold_block = [&](int64_t b, const RawN<T, DPL>* zc, const RawN<T, DPL>* xc) {
    // block maximum of z (log2 units): the reference of this block's sums
    float bmx[DPL];
#pragma unroll
    for (int d = 0; d < DPL; ++d) {
      float v = zc[0][d];
#pragma unroll
      for (int t = 1; t < M; ++t) v = fmaxf(v, zc[t][d]);
      bmx[d] = v * L2E;
    }
    float sA[DPL], aA[DPL], sB[DPL], aB[DPL];
#pragma unroll
    for (int d = 0; d < DPL; ++d) { sA[d] = 0.f; aA[d] = 0.f; sB[d] = 0.f; aB[d] = 0.f; }
#pragma unroll
    for (int t = 0; t < M; ++t) {
      float ba[DPL], bb[DPL];
#pragma unroll
      for (int d = 0; d < DPL; d += 4) {
        const float4 va = *reinterpret_cast<const float4*>(&beta[t][d0 + d]);
        const float4 vb = *reinterpret_cast<const float4*>(&beta[M + t][d0 + d]);
        ba[d] = va.x; ba[d + 1] = va.y; ba[d + 2] = va.z; ba[d + 3] = va.w;
        bb[d] = vb.x; bb[d + 1] = vb.y; bb[d + 2] = vb.z; bb[d + 3] = vb.w;
      }
#pragma unroll
      for (int d = 0; d < DPL; ++d) {
        const float u = __builtin_amdgcn_exp2f(fmaf(zc[t][d], L2E, -bmx[d]));
        const float xv = xc[t][d];
        const float wa = u * ba[d];
        const float wb = u * bb[d];
        sA[d] += wa;
        aA[d] = fmaf(wa, xv, aA[d]);
        sB[d] += wb;
        aB[d] = fmaf(wb, xv, aB[d]);
      }
      asm volatile("" ::: "memory");           // fold token by token (register pressure)
    }
    {                                          // this block closes entry b
      float o[DPL];
      const bool first = b == 0;               // entry 0 has no previous block
#pragma unroll
      for (int d = 0; d < DPL; ++d) {
        // join the two halves at the larger of their references
        const float dl = cr[d] - bmx[d];
        const float g = __builtin_amdgcn_exp2f(-fabsf(dl));
        const float fc = first ? 0.f : (dl >= 0.f ? 1.f : g);
        const float fb = (first || dl < 0.f) ? 1.f : g;
        o[d] = (cA[d] * fc + aB[d] * fb) * __builtin_amdgcn_rcpf(cS[d] * fc + sB[d] * fb);
      }
      // rows outside [e0, e1) fall past the buffer record and are dropped
      const uint32_t off = (b >= e0 && b < e1) ? (uint32_t)((b - e0) * ld_out + d0) * sizeof(T)
                                               : 0xffffffffu;
      BufStoreN<T, DPL>::store(orsrc, off, o);
    }
#pragma unroll
    for (int d = 0; d < DPL; ++d) { cS[d] = sA[d]; cA[d] = aA[d]; cr[d] = bmx[d]; }
  };
#pragma unroll
  for (int i = 0; i < kRing - 1; ++i) load_block(bk + i, zb[i], xb[i]);
  // whole rounds of kRing blocks; folds past e1 compute on re-read data and
  // store nothing
  for (; bk < e1; bk += kRing) {
#pragma unroll
    for (int i = 0; i < kRing; ++i) {
      const int nx = (i + kRing - 1) % kRing;
      load_block(bk + i + kRing - 1, zb[nx], xb[nx]);
      fold_block(bk + i, zb[i], xb[i]);
    }
  }
}

// ---------------------------------------------------------------------------
// Streaming compressor for large blocks (m > 4), the HCA scale.
//
// The bias goes inside the exponent: w = 2^((z + b_p) * log2e - r), so no
// per-position table is needed (the 2m x 512 bias rows stay in L2).  Each
// half window has its own reference r, set by the first chunk of the block
// and raised only when a chunk maximum exceeds r + kBand; the two halves of
// an entry are joined with an exact rescale to the larger reference.
//
// A block of kLargeWaves waves covers consecutive entry ranges of one dim
// slice.  Wave w streams its own range; the first half of its first entry
// comes from the last block of wave w-1, so each wave keeps that entry's
// second half aside and the halves are joined through LDS after a barrier.
// Wave 0 reads the one block before the range itself and gets one entry
// less, so every wave streams the same number of blocks.
#ifndef CSKV_LARGE_WAVES
#define CSKV_LARGE_WAVES 8
#endif
constexpr int kLargeWaves = CSKV_LARGE_WAVES;
#ifndef CSKV_LARGE_DPL
#define CSKV_LARGE_DPL 4
#endif
#ifndef CSKV_LARGE_EPW
#define CSKV_LARGE_EPW 4
#endif
constexpr int kLargeDpl = CSKV_LARGE_DPL;
constexpr int kLargeEpw = CSKV_LARGE_EPW;   // entries per wave (wave 0: one less)
#ifndef CSKV_LARGE_CHUNK
#define CSKV_LARGE_CHUNK 4
#endif
constexpr int kLargeChunk = CSKV_LARGE_CHUNK;   // tokens per chunk (register block)

template <class T, int DPL>
__global__ __launch_bounds__(64 * kLargeWaves) void compress_large_kernel(
    const T* __restrict__ x, const T* __restrict__ z, const float* __restrict__ bias, int m,
    int64_t e_begin, int64_t e_end, int epw, T* __restrict__ out, int64_t ld_out) {
  constexpr int kSlices = kD / (64 * DPL);
  constexpr int C = kLargeChunk;
  __shared__ float xch[kLargeWaves][3][kD];        // carried half of each wave's last block
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int blk = xcd_contiguous(blockIdx.x, gridDim.x);
  const int slice = blk % kSlices;
  const int64_t group = blk / kSlices;
  const int d0 = slice * 64 * DPL + lane * DPL;
  const float L2E = 1.4426950408889634f;
  // entries of this block: [g0, g0 + kLargeWaves*epw - 1); wave 0 gets epw-1
  const int64_t g0 = e_begin + group * ((int64_t)kLargeWaves * epw - 1);
  const int64_t e0 = wave == 0 ? g0 : g0 + (int64_t)wave * epw - 1;
  const int64_t e1r = g0 + (int64_t)(wave + 1) * epw - 1;
  const int64_t e1 = e1r < e_end ? e1r : e_end;
  // wave 0 streams the block before its range (unless it is the first)
  const int64_t b_first = (wave == 0 && e0 > 0) ? e0 - 1 : e0;

  // Each half window keeps its own reference (log2 units), raised lazily
  // within the block: rA for the first half of entry b+1, rB for the second
  // half of entry b.  cS/cA/cr: carried first half of the current entry.
  float cS[DPL], cA[DPL], cr[DPL];
  float fS[DPL], fA[DPL], fr[DPL];           // second half of the first entry (waves > 0)
#pragma unroll
  for (int d = 0; d < DPL; ++d) {
    cS[d] = 0.f; cA[d] = 0.f; cr[d] = 0.f; fS[d] = 0.f; fA[d] = 0.f; fr[d] = 0.f;
  }
  for (int64_t b = b_first; b < e1; ++b) {
    float sA[DPL], aA[DPL], sB[DPL], aB[DPL], rA[DPL], rB[DPL];
#pragma unroll
    for (int d = 0; d < DPL; ++d) { sA[d] = 0.f; aA[d] = 0.f; sB[d] = 0.f; aB[d] = 0.f; }
    for (int t0 = 0; t0 < m; t0 += C) {
      RawN<T, DPL> zc[C], xc[C];
      float lA[C][DPL], lB[C][DPL];
#pragma unroll
      for (int t = 0; t < C; ++t) {
        if (t0 + t < m) {
          const int64_t j = b * m + t0 + t;
          zc[t].load(z + j * kD + d0);
          xc[t].load(x + j * kD + d0);
#pragma unroll
          for (int d = 0; d < DPL; d += 4) {
            const float4 va = *reinterpret_cast<const float4*>(bias + (int64_t)(t0 + t) * kD + d0 + d);
            const float4 vb = *reinterpret_cast<const float4*>(bias + (int64_t)(m + t0 + t) * kD + d0 + d);
            lA[t][d] = va.x; lA[t][d + 1] = va.y; lA[t][d + 2] = va.z; lA[t][d + 3] = va.w;
            lB[t][d] = vb.x; lB[t][d + 1] = vb.y; lB[t][d + 2] = vb.z; lB[t][d + 3] = vb.w;
          }
        }
      }
      // logits in log2 units and the chunk maxima of each half
      float mA[DPL], mB[DPL];
#pragma unroll
      for (int d = 0; d < DPL; ++d) { mA[d] = -INFINITY; mB[d] = -INFINITY; }
#pragma unroll
      for (int t = 0; t < C; ++t) {
#pragma unroll
        for (int d = 0; d < DPL; ++d) {
          const bool ok = t0 + t < m;
          const float zv = zc[t][d];
          lA[t][d] = ok ? (zv + lA[t][d]) * L2E : -INFINITY;
          lB[t][d] = ok ? (zv + lB[t][d]) * L2E : -INFINITY;
          mA[d] = fmaxf(mA[d], lA[t][d]);
          mB[d] = fmaxf(mB[d], lB[t][d]);
        }
      }
      if (t0 == 0) {
#pragma unroll
        for (int d = 0; d < DPL; ++d) { rA[d] = mA[d]; rB[d] = mB[d]; }
      } else {
        bool up = false;
#pragma unroll
        for (int d = 0; d < DPL; ++d) up |= (mA[d] > rA[d] + kBand) || (mB[d] > rB[d] + kBand);
        if (__any(up)) {
#pragma unroll
          for (int d = 0; d < DPL; ++d) {
            const float na = mA[d] > rA[d] + kBand ? mA[d] : rA[d];
            const float nb = mB[d] > rB[d] + kBand ? mB[d] : rB[d];
            const float fa = __builtin_amdgcn_exp2f(rA[d] - na);
            const float fb = __builtin_amdgcn_exp2f(rB[d] - nb);
            sA[d] *= fa; aA[d] *= fa; sB[d] *= fb; aB[d] *= fb;
            rA[d] = na; rB[d] = nb;
          }
        }
      }
#pragma unroll
      for (int t = 0; t < C; ++t) {
#pragma unroll
        for (int d = 0; d < DPL; ++d) {
          const float xv = xc[t][d];
          const float wa = __builtin_amdgcn_exp2f(lA[t][d] - rA[d]);
          const float wb = __builtin_amdgcn_exp2f(lB[t][d] - rB[d]);
          sA[d] += wa;
          aA[d] = fmaf(wa, xv, aA[d]);
          sB[d] += wb;
          aB[d] = fmaf(wb, xv, aB[d]);
        }
      }
    }
    // block b closes entry b (second half here, first half carried)
    if (b >= e0) {
      if (b == e0 && wave > 0) {
        // first half of this entry comes from wave-1: keep the second half aside
#pragma unroll
        for (int d = 0; d < DPL; ++d) { fS[d] = sB[d]; fA[d] = aB[d]; fr[d] = rB[d]; }
      } else {
        float o[DPL];
        const bool first = b == 0;             // entry 0 has no first half
#pragma unroll
        for (int d = 0; d < DPL; ++d) {
          const float mx = fmaxf(cr[d], rB[d]);
          const float fc = first ? 0.f : __builtin_amdgcn_exp2f(cr[d] - mx);
          const float fb = __builtin_amdgcn_exp2f(rB[d] - mx);
          o[d] = (cA[d] * fc + aB[d] * fb) * __builtin_amdgcn_rcpf(cS[d] * fc + sB[d] * fb);
        }
        StoreN<T, DPL>::store(out + b * ld_out + d0, o);
      }
    }
#pragma unroll
    for (int d = 0; d < DPL; ++d) { cS[d] = sA[d]; cA[d] = aA[d]; cr[d] = rA[d]; }
  }
  // hand the carried first half to the next wave
#pragma unroll
  for (int d = 0; d < DPL; ++d) {
    xch[wave][0][lane * DPL + d] = cS[d];
    xch[wave][1][lane * DPL + d] = cA[d];
    xch[wave][2][lane * DPL + d] = cr[d];
  }
  __syncthreads();
  if (wave > 0 && e0 < e1) {
    float o[DPL];
#pragma unroll
    for (int d = 0; d < DPL; ++d) {
      const float pS = xch[wave - 1][0][lane * DPL + d];
      const float pA = xch[wave - 1][1][lane * DPL + d];
      const float pr = xch[wave - 1][2][lane * DPL + d];
      const float mx = fmaxf(pr, fr[d]);
      const float fp = __builtin_amdgcn_exp2f(pr - mx), fc = __builtin_amdgcn_exp2f(fr[d] - mx);
      o[d] = (pA * fp + fA[d] * fc) * __builtin_amdgcn_rcpf(pS * fp + fS[d] * fc);
    }
    StoreN<T, DPL>::store(out + e0 * ld_out + d0, o);
  }
}

template <class T>
static hipError_t launch_large_t(const void* x, const void* z, const float* bias, int m,
                                 int64_t e_begin, int64_t e_end, void* out, int64_t ld_out,
                                 hipStream_t stream) {
  constexpr int kSlices = kD / (64 * kLargeDpl);
  const int64_t n = e_end - e_begin;
  const int64_t per = (int64_t)kLargeWaves * kLargeEpw - 1;   // entries per block of waves
  const int64_t groups = (n + per - 1) / per;
  hipLaunchKernelGGL((compress_large_kernel<T, kLargeDpl>), dim3((unsigned)(groups * kSlices)),
                     dim3(64 * kLargeWaves), 0, stream, (const T*)x, (const T*)z, bias, m, e_begin,
                     e_end, kLargeEpw, (T*)out, ld_out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Fused two-scale compressor: one pass over x and z produces the entries of
// a small block size MS (<= 4, the CSA scale) and of a large block size ML =
// R * MS <= 128 (the HCA scale), since both read the same raw rows.
//
// Weights share one exp2 per element: with r the maximum of z over the small
// block being read (per dimension),
//   small window:  2^(z*log2e - r) * beta_s[p],   beta_s = 2^((b_s - max b_s) log2e)
//   large window:  2^(z*log2e - r) * beta_l[p],   beta_l = 2^((b_l - max b_l) log2e)
// (the constant factors cancel in each normalisation).  With ux = u x every
// accumulation is one FMA.  A block takes 128 dimensions (2 per lane), so
// that both weight tables of its dimensions fit LDS whole (beta_l: 2*ML rows,
// 128 KB at ML = 128, computed by the block from the bias before it
// streams): the 16 waves stream
// their ranges with no barrier.  A small block's large sums join the running
// sums of its large block once, scaled by 2^(r - rl) with rl the large
// block's raise-only reference.  Wave ranges hand their carried halves to the
// next wave through LDS; the first wave of a block leaves its deferred halves,
// and the last wave its carried ones, in the workspace for the join kernel.

// One entry from its two half-window sums, each with its own reference
// (log2 domain): both are brought to the larger reference.
__device__ __forceinline__ float join_halves(float pS, float pA, float pr, float sS, float sA, float sr) {
  const float mx = fmaxf(pr, sr);
  const float fp = __builtin_amdgcn_exp2f(pr - mx), fc = __builtin_amdgcn_exp2f(sr - mx);
  return (pA * fp + sA * fc) * __builtin_amdgcn_rcpf(pS * fp + sS * fc);
}
__device__ __forceinline__ void store_elem(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_elem(bf16_t* p, float v) { p->u = (uint16_t)f32_to_bf16(v); }

constexpr int kFusedWaves = 16;                // one block of 1024 threads per CU
constexpr int kFusedDpl = 2;                   // dimensions per lane
constexpr int kFusedSW = 64 * kFusedDpl;       // dimensions per block
constexpr int kFusedSlices = kD / kFusedSW;
constexpr int kFusedMaxML = 128;               // largest large block whose weights fit LDS

template <class T, int MS>
__global__ __launch_bounds__(64 * kFusedWaves) void compress_fused_kernel(
    const T* __restrict__ x, const T* __restrict__ z, const float* __restrict__ bias_s,
    const float* __restrict__ bias_l, int R, int64_t NL, int epw, T* __restrict__ out_s,
    int64_t ld_s, T* __restrict__ out_l, int64_t ld_l, float* __restrict__ bnd) {
  constexpr int DPL = kFusedDpl, kSW = kFusedSW;
  const int ML = R * MS;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int blk = xcd_contiguous(blockIdx.x, gridDim.x);
  const int slice = blk % kFusedSlices;
  const int64_t group = blk / kFusedSlices;
  const int dl = lane * DPL;                      // dim within the slice
  const int d0 = slice * kSW + dl;
  const float L2E = 1.4426950408889634f;
  // large entries of this wave: [E0, E1), streamed as large blocks from E0
  const int64_t E0 = (group * kFusedWaves + wave) * (int64_t)epw;
  const int64_t E1 = E0 + epw < NL ? E0 + epw : NL;
  const int nblocks = epw;                        // large blocks streamed by every wave
  // the first entries of a range wait for the previous range's carried
  // halves: through LDS inside the block, through the workspace (and the
  // join kernel) across blocks; entry 0 has no first half
  const bool deferred = wave > 0 || group > 0;
  const int64_t NS = NL * R;                      // small entries
  const int64_t S0 = E0 * R, S1 = E1 * R;         // small entries written by this wave

  // both weight tables of this block's dimensions; after the loop the
  // large table's space takes the waves' carried halves
  __shared__ __attribute__((aligned(16))) float bl_lds[2 * kFusedMaxML][kSW];
  __shared__ __attribute__((aligned(16))) float bs_lds[2 * MS][kSW];
  static_assert(kFusedWaves * 6 <= 2 * kFusedMaxML, "carried halves fit the table's space");
  float(*xch)[6][kSW] = reinterpret_cast<float(*)[6][kSW]>(&bl_lds[0][0]);
  for (int i = threadIdx.x; i < 2 * MS * kSW; i += 64 * kFusedWaves) {
    const int p = i / kSW, d = i % kSW;
    float bm = bias_s[slice * kSW + d];
    for (int q = 1; q < 2 * MS; ++q) bm = fmaxf(bm, bias_s[(int64_t)q * kD + slice * kSW + d]);
    bs_lds[p][d] = __builtin_amdgcn_exp2f((bias_s[(int64_t)p * kD + slice * kSW + d] - bm) * L2E);
  }
  // the large scale's weights beta_l[p][d] = 2^((b[p][d] - max_p b[p][d]) log2e)
  // of this block's dimensions: thread t takes dimension t % kSW and the
  // rows of row group t / kSW (every kRG-th row), so each row load is one
  // coalesced 512-byte run; the group maxima meet in LDS
  {
    constexpr int kRG = 64 * kFusedWaves / kSW;              // row groups (8)
    constexpr int kRows = 2 * kFusedMaxML / kRG;             // rows a thread takes, at most (32)
    __shared__ float gmx[kRG][kSW];
    const int dd = threadIdx.x % kSW, rg = threadIdx.x / kSW;
    const float* bcol = bias_l + slice * kSW + dd;
    float bv[kRows];
    float bm = -INFINITY;
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
      const int p = rg + kRG * i;
      bv[i] = p < 2 * ML ? bcol[(int64_t)p * kD] : -INFINITY;
      bm = fmaxf(bm, bv[i]);
    }
    gmx[rg][dd] = bm;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kRG; ++i) bm = fmaxf(bm, gmx[i][dd]);
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
      const int p = rg + kRG * i;
      if (p < 2 * ML) bl_lds[p][dd] = __builtin_amdgcn_exp2f((bv[i] - bm) * L2E);
    }
  }

  // Small scale: carried first half cS/cA of the next entry with its
  // reference cr (the maximum of the block it came from).  Large scale:
  // reference rl of the current large block (raise-only within the block;
  // both halves of the block use it), running halves lsA/laA, lsB/laB, and
  // the carried first half lcS/lcA of the next large entry with its
  // reference lcr.  f*/g*: the deferred second halves of the range's first
  // small and large entries.
  float cS[DPL], cA[DPL], cr[DPL];
  float rl[DPL], lcS[DPL], lcA[DPL], lcr[DPL];
  float lsA[DPL], laA[DPL], lsB[DPL], laB[DPL];
  float fS[DPL], fA[DPL], fR[DPL], gS[DPL], gA[DPL], gR[DPL];
#pragma unroll
  for (int d = 0; d < DPL; ++d) {
    cr[d] = 0.f; cS[d] = cA[d] = 0.f;
    rl[d] = -INFINITY; lcS[d] = lcA[d] = lcr[d] = 0.f;
    lsA[d] = laA[d] = lsB[d] = laB[d] = 0.f;
    fS[d] = fA[d] = fR[d] = gS[d] = gA[d] = gR[d] = 0.f;
  }
  const int64_t sbegin = E0 * R;                             // first small block streamed
  const int64_t sb_last = NS - 1;                            // last small block inside NL large blocks
  auto load_sb = [&](int64_t sb, RawN<T, DPL>* zz, RawN<T, DPL>* xx) {
    if (sb > sb_last) sb = sb_last;
#pragma unroll
    for (int t = 0; t < MS; ++t) {
      const int64_t j = sb * MS + t;
      zz[t].load_nt(z + j * kD + d0);                        // read once: no cache allocation
      xx[t].load_nt(x + j * kD + d0);
    }
  };
  const __amdgpu_buffer_rsrc_t rsrc_s =
      make_rsrc(out_s + (S0 < S1 ? S0 : 0) * ld_s, S0 < S1 ? (uint32_t)((S1 - S0) * ld_s * sizeof(T)) : 0u);
  const __amdgpu_buffer_rsrc_t rsrc_l =
      make_rsrc(out_l + (E0 < E1 ? E0 : 0) * ld_l, E0 < E1 ? (uint32_t)((E1 - E0) * ld_l * sizeof(T)) : 0u);

  // Two register slots of raw rows: the step reading one loads the next
  // block into the other.  A wave streams its large blocks in an outer loop
  // and their R (even) small blocks in an inner loop unrolled by two, so that
  // the slots are fixed per unrolled step and a large entry closes outside
  // the inner loop.
  RawN<T, DPL> zb[2][MS], xb[2][MS];
  load_sb(sbegin, zb[0], xb[0]);
  __syncthreads();                                           // weight tables ready

  // small block j of large block bi (global small block sb); lp = j * MS is
  // its first position in the large window's first half
  auto step = [&](const int64_t sb, const int lp, const RawN<T, DPL>* zc, const RawN<T, DPL>* xc,
                  RawN<T, DPL>* zn, RawN<T, DPL>* xn) {
    load_sb(sb + 1, zn, xn);
    // reference from the small block maximum
    float bmx[DPL];
#pragma unroll
    for (int d = 0; d < DPL; ++d) {
      float v = zc[0][d];
#pragma unroll
      for (int t = 1; t < MS; ++t) v = fmaxf(v, zc[t][d]);
      bmx[d] = v * L2E;
    }
    // This block's sums, all against its maximum bmx: the small halves
    // (sA/aA: first half of entry sb + 1, sB/aB: second half of entry
    // sb) and the large block's two halves (pA/qA, pB/qB).
    float sA[DPL], aA[DPL], sB[DPL], aB[DPL], pA[DPL], qA[DPL], pB[DPL], qB[DPL];
#pragma unroll
    for (int t = 0; t < MS; ++t) {
      const float2 ba = *reinterpret_cast<const float2*>(&bs_lds[t][dl]);
      const float2 bb = *reinterpret_cast<const float2*>(&bs_lds[MS + t][dl]);
      const float2 la = *reinterpret_cast<const float2*>(&bl_lds[lp + t][dl]);
      const float2 lb = *reinterpret_cast<const float2*>(&bl_lds[ML + lp + t][dl]);
#pragma unroll
      for (int d = 0; d < DPL; ++d) {
        const float wa = d ? ba.y : ba.x, wb = d ? bb.y : bb.x;
        const float va = d ? la.y : la.x, vb = d ? lb.y : lb.x;
        const float u = __builtin_amdgcn_exp2f(fmaf(zc[t][d], L2E, -bmx[d]));
        const float ux = u * xc[t][d];
        if (t == 0) {
          sA[d] = u * wa; aA[d] = ux * wa; sB[d] = u * wb; aB[d] = ux * wb;
          pA[d] = u * va; qA[d] = ux * va; pB[d] = u * vb; qB[d] = ux * vb;
        } else {
          sA[d] = fmaf(u, wa, sA[d]);
          aA[d] = fmaf(ux, wa, aA[d]);
          sB[d] = fmaf(u, wb, sB[d]);
          aB[d] = fmaf(ux, wb, aB[d]);
          pA[d] = fmaf(u, va, pA[d]);
          qA[d] = fmaf(ux, va, qA[d]);
          pB[d] = fmaf(u, vb, pB[d]);
          qB[d] = fmaf(ux, vb, qB[d]);
        }
      }
    }
    // The large block's reference rl is raise-only within the block (it
    // is -inf before the block's first small block); this block's large sums
    // join the running sums scaled by G = 2^(bmx - rl) <= 2^kBand.  Raising
    // rl (rare, and at every large block's start) rescales the running sums.
    bool up = false;
#pragma unroll
    for (int d = 0; d < DPL; ++d) up |= bmx[d] > rl[d] + kBand;
    if (__any(up)) {
#pragma unroll
      for (int d = 0; d < DPL; ++d) {
        const float na = bmx[d] > rl[d] + kBand ? bmx[d] : rl[d];
        const float f = __builtin_amdgcn_exp2f(rl[d] - na);
        lsA[d] *= f; laA[d] *= f; lsB[d] *= f; laB[d] *= f;
        rl[d] = na;
      }
    }
#pragma unroll
    for (int d = 0; d < DPL; ++d) {
      const float G = __builtin_amdgcn_exp2f(bmx[d] - rl[d]);
      lsA[d] = fmaf(G, pA[d], lsA[d]);
      laA[d] = fmaf(G, qA[d], laA[d]);
      lsB[d] = fmaf(G, pB[d], lsB[d]);
      laB[d] = fmaf(G, qB[d], laB[d]);
    }
    // small entry sb: carried first half + this second half
    float o[DPL];
    const bool first = sb == 0;
#pragma unroll
    for (int d = 0; d < DPL; ++d) {
      const float dl2 = cr[d] - bmx[d];
      const float g = __builtin_amdgcn_exp2f(-fabsf(dl2));
      const float fc = first ? 0.f : (dl2 >= 0.f ? 1.f : g);
      const float fb = (first || dl2 < 0.f) ? 1.f : g;
      o[d] = (cA[d] * fc + aB[d] * fb) * __builtin_amdgcn_rcpf(cS[d] * fc + sB[d] * fb);
    }
    const bool defer = deferred && sb == S0;                 // first half comes from the previous range
    if (defer) {
#pragma unroll
      for (int d = 0; d < DPL; ++d) { fS[d] = sB[d]; fA[d] = aB[d]; fR[d] = bmx[d]; }
    }
    const uint32_t off = (sb >= S0 && sb < S1 && !defer)
                             ? (uint32_t)((sb - S0) * ld_s + d0) * sizeof(T) : 0xffffffffu;
    BufStoreN<T, DPL>::store(rsrc_s, off, o);
#pragma unroll
    for (int d = 0; d < DPL; ++d) { cS[d] = sA[d]; cA[d] = aA[d]; cr[d] = bmx[d]; }
  };

  for (int bi = 0; bi < nblocks; ++bi) {
    const int64_t lb = E0 + bi;                              // large block
    for (int j = 0; j < R; j += 2) {
      step(lb * R + j, j * MS, zb[0], xb[0], zb[1], xb[1]);
      step(lb * R + j + 1, (j + 1) * MS, zb[1], xb[1], zb[0], xb[0]);
    }
    // end of a large block: large entry lb closes
    float o[DPL];
    const bool first = lb == 0;
#pragma unroll
    for (int d = 0; d < DPL; ++d) {
      const float mx = fmaxf(lcr[d], rl[d]);
      const float fc = first ? 0.f : __builtin_amdgcn_exp2f(lcr[d] - mx);
      const float fb = __builtin_amdgcn_exp2f(rl[d] - mx);
      o[d] = (lcA[d] * fc + laB[d] * fb) * __builtin_amdgcn_rcpf(lcS[d] * fc + lsB[d] * fb);
    }
    const bool defer = deferred && lb == E0;
    if (defer) {
#pragma unroll
      for (int d = 0; d < DPL; ++d) { gS[d] = lsB[d]; gA[d] = laB[d]; gR[d] = rl[d]; }
    }
    const uint32_t off = (lb >= E0 && lb < E1 && !defer)
                             ? (uint32_t)((lb - E0) * ld_l + d0) * sizeof(T) : 0xffffffffu;
    BufStoreN<T, DPL>::store(rsrc_l, off, o);
#pragma unroll
    for (int d = 0; d < DPL; ++d) {
      lcS[d] = lsA[d]; lcA[d] = laA[d]; lcr[d] = rl[d];
      lsA[d] = 0.f; laA[d] = 0.f; lsB[d] = 0.f; laB[d] = 0.f;
      rl[d] = -INFINITY;
    }
  }
  // hand both carried first halves (and the references) to the next wave;
  // the last wave's go to the workspace for the next block's first wave,
  // which leaves its deferred halves there too
  __syncthreads();                                           // every wave is done with the tables
#pragma unroll
  for (int d = 0; d < DPL; ++d) {
    xch[wave][0][dl + d] = cS[d];
    xch[wave][1][dl + d] = cA[d];
    xch[wave][2][dl + d] = lcS[d];
    xch[wave][3][dl + d] = lcA[d];
    xch[wave][4][dl + d] = cr[d];
    xch[wave][5][dl + d] = lcr[d];
  }
  float* bg = bnd + group * (int64_t)(12 * kD);
  if (wave == kFusedWaves - 1) {
#pragma unroll
    for (int d = 0; d < DPL; ++d) {
      bg[0 * kD + d0 + d] = cS[d];
      bg[1 * kD + d0 + d] = cA[d];
      bg[2 * kD + d0 + d] = cr[d];
      bg[3 * kD + d0 + d] = lcS[d];
      bg[4 * kD + d0 + d] = lcA[d];
      bg[5 * kD + d0 + d] = lcr[d];
    }
  }
  if (wave == 0 && group > 0) {
#pragma unroll
    for (int d = 0; d < DPL; ++d) {
      bg[6 * kD + d0 + d] = fS[d];
      bg[7 * kD + d0 + d] = fA[d];
      bg[8 * kD + d0 + d] = fR[d];
      bg[9 * kD + d0 + d] = gS[d];
      bg[10 * kD + d0 + d] = gA[d];
      bg[11 * kD + d0 + d] = gR[d];
    }
  }
  __syncthreads();
  if (wave > 0) {
    float os[DPL], ol[DPL];
#pragma unroll
    for (int d = 0; d < DPL; ++d) {
      os[d] = join_halves(xch[wave - 1][0][dl + d], xch[wave - 1][1][dl + d], xch[wave - 1][4][dl + d],
                          fS[d], fA[d], fR[d]);
      ol[d] = join_halves(xch[wave - 1][2][dl + d], xch[wave - 1][3][dl + d], xch[wave - 1][5][dl + d],
                          gS[d], gA[d], gR[d]);
    }
    BufStoreN<T, DPL>::store(rsrc_s, S0 < S1 ? (uint32_t)(d0 * sizeof(T)) : 0xffffffffu, os);
    BufStoreN<T, DPL>::store(rsrc_l, E0 < E1 ? (uint32_t)(d0 * sizeof(T)) : 0xffffffffu, ol);
  }
}

// The first small and large entries of every block but the first: the
// previous block's carried first halves joined with this block's deferred
// second halves (both in the workspace).  One thread per dimension.
template <class T>
__global__ __launch_bounds__(256) void compress_join_kernel(const float* __restrict__ bnd, int64_t groups,
                                                            int per, int R, int64_t NL,
                                                            T* __restrict__ out_s, int64_t ld_s,
                                                            T* __restrict__ out_l, int64_t ld_l) {
  const int64_t g = 1 + blockIdx.x / (kD / 256);
  const int d = (blockIdx.x % (kD / 256)) * 256 + threadIdx.x;
  const int64_t E = g * per;                                 // the block's first large entry
  if (g >= groups || E >= NL) return;
  const float* c = bnd + (g - 1) * (int64_t)(12 * kD);       // carried by the previous block
  const float* f = bnd + g * (int64_t)(12 * kD);             // deferred by this block
  const float os = join_halves(c[0 * kD + d], c[1 * kD + d], c[2 * kD + d],
                               f[6 * kD + d], f[7 * kD + d], f[8 * kD + d]);
  const float ol = join_halves(c[3 * kD + d], c[4 * kD + d], c[5 * kD + d],
                               f[9 * kD + d], f[10 * kD + d], f[11 * kD + d]);
  store_elem(out_s + (E * R) * ld_s + d, os);
  store_elem(out_l + E * ld_l + d, ol);
}

template <class T>
static hipError_t launch_fused_t(const void* x, const void* z, int64_t T_tokens, const float* bias_s,
                                 int ms, void* out_s, int64_t ld_s, const float* bias_l, int ml,
                                 void* out_l, int64_t ld_l, void* ws, hipStream_t stream) {
  const int64_t NL = T_tokens / ml;
  const int R = ml / ms;
  float* bnd = (float*)ws;                                   // per block: 12 x 512 boundary halves
  const T* xp = (const T*)x;
  const T* zp = (const T*)z;
  int epw = 2;
  int64_t groups = 0;
  auto pick = [&](const void* kern) {
    // Large entries per wave: the grid runs in rounds of the blocks that fit
    // on the chip at once; take the epw (at least 1) that fills its last
    // round best, the largest of equals (fewest block boundaries to join).
    // The resident block count is queried on every call, for the current
    // device (host-side queries, no device work, nothing kept between calls).
    int nb = 0, dev = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kern, 64 * kFusedWaves, 0) != hipSuccess ||
        hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      nb = 0;
    const int slots = nb > 0 && cus > 0 ? nb * cus : 256;
    double best = -1.0;
    for (int e = 1; e <= 64; ++e) {
      const int64_t per = (int64_t)kFusedWaves * e;
      const int64_t g = (NL + per - 1) / per;
      const double rounds = (double)(g * kFusedSlices) / slots;
      const double eff = rounds / std::ceil(rounds) * (double)NL / (double)(g * per);
      if (eff >= best - 1e-9) { best = eff; epw = e; groups = g; }
    }
  };
#define CSKV_FUSED(MS)                                                                            \
  pick((const void*)compress_fused_kernel<T, MS>);                                            \
  hipLaunchKernelGGL((compress_fused_kernel<T, MS>), dim3((unsigned)(groups * kFusedSlices)),     \
                     dim3(64 * kFusedWaves), 0, stream, xp, zp, bias_s, bias_l, R, NL, epw,        \
                     (T*)out_s, ld_s, (T*)out_l, ld_l, bnd)
  switch (ms) {
    case 1: CSKV_FUSED(1); break;
    case 2: CSKV_FUSED(2); break;
    case 3: CSKV_FUSED(3); break;
    default: CSKV_FUSED(4); break;
  }
#undef CSKV_FUSED
  if (groups > 1)
    hipLaunchKernelGGL(compress_join_kernel<T>, dim3((unsigned)((groups - 1) * (kD / 256))), dim3(256), 0,
                       stream, bnd, groups, kFusedWaves * epw, R, NL, (T*)out_s, ld_s, (T*)out_l, ld_l);
  return hipGetLastError();
}

hipError_t launch_compress_fused(int dt, const void* x, const void* z, int64_t T_tokens,
                                 const float* bias_s, int ms, void* out_s, int64_t ld_s,
                                 const float* bias_l, int ml, void* out_l, int64_t ld_l, void* ws,
                                 hipStream_t stream) {
  const int64_t NL = T_tokens / ml, NSall = T_tokens / ms, NSf = NL * (ml / ms);
  hipError_t e = hipSuccess;
  if ((ml / ms) % 2 != 0 || ml > kFusedMaxML) {
    // the fused kernel streams an even number of small blocks per large
    // block and holds the large scale's weights in LDS (ml <= 128);
    // otherwise each scale gets its own streaming kernel
    e = launch_compress(dt, x, z, bias_s, ms, 0, NSall, out_s, ld_s, stream);
    if (e == hipSuccess && NL > 0) e = launch_compress(dt, x, z, bias_l, ml, 0, NL, out_l, ld_l, stream);
    return e;
  }
  if (NL > 0) {
    e = dt == 0 ? launch_fused_t<float>(x, z, T_tokens, bias_s, ms, out_s, ld_s, bias_l, ml, out_l,
                                        ld_l, ws, stream)
                : launch_fused_t<bf16_t>(x, z, T_tokens, bias_s, ms, out_s, ld_s, bias_l, ml, out_l,
                                         ld_l, ws, stream);
    if (e != hipSuccess) return e;
  }
  // small entries past the last whole large block
  if (NSall > NSf) e = launch_compress(dt, x, z, bias_s, ms, NSf, NSall, out_s, ld_s, stream);
  return e;
}

// The pooling-weight table plus the boundary halves of every block (at
// most one block per 2 * kFusedWaves large entries).
size_t compress_fused_workspace_bytes(int64_t T_tokens, int ml) {
  const int64_t NL = T_tokens / ml;
  const int64_t groups = (NL + kFusedWaves - 1) / kFusedWaves;  // at one large block a wave, the most
  (void)ml;
  return (size_t)groups * 12 * kD * sizeof(float) + 256;
}

template <class T>
static hipError_t launch_small_t(const void* x, const void* z, const float* bias, int m,
                                 int64_t e_begin, int64_t e_end, void* out, int64_t ld_out,
                                 hipStream_t stream) {
  constexpr int DPL = kSmallDpl;
  constexpr int kSlices = kD / (64 * DPL);
  const int64_t n = e_end - e_begin;
  int64_t epw = n / kSmallRanges;
  epw = epw < 8 ? 8 : (epw > 256 ? 256 : epw);
  const int64_t waves = (n + epw - 1) / epw * kSlices;
  const int64_t grid = (waves + 3) / 4;
  const T* xp = (const T*)x;
  const T* zp = (const T*)z;
  T* op = (T*)out;
#define CSKV_SMALL(M)                                                                           \
  hipLaunchKernelGGL((compress_small_kernel<T, M, DPL>), dim3((unsigned)grid), dim3(256), 0, stream, \
                     xp, zp, bias, e_begin, e_end, (int)epw, op, ld_out)
  switch (m) {
    case 1: CSKV_SMALL(1); break;
    case 2: CSKV_SMALL(2); break;
    case 3: CSKV_SMALL(3); break;
    default: CSKV_SMALL(4); break;
  }
#undef CSKV_SMALL
  return hipGetLastError();
}

hipError_t launch_compress(int dt, const void* x, const void* z, const float* bias, int m,
                           int64_t e_begin, int64_t e_end, void* out, int64_t ld_out,
                           hipStream_t stream) {
  if (e_end <= e_begin) return hipSuccess;
  if (m <= 4) {
    if (dt == 0) return launch_small_t<float>(x, z, bias, m, e_begin, e_end, out, ld_out, stream);
    return launch_small_t<bf16_t>(x, z, bias, m, e_begin, e_end, out, ld_out, stream);
  }
  if (dt == 0) return launch_large_t<float>(x, z, bias, m, e_begin, e_end, out, ld_out, stream);
  return launch_large_t<bf16_t>(x, z, bias, m, e_begin, e_end, out, ld_out, stream);
}

}  // namespace cskv
