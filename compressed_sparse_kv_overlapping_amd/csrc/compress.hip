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

// ---------------------------------------------------------------------------
// Streaming compressor for small blocks (m <= 4), the CSA scale.
//
// A wave streams a contiguous range of entries and reads every token once.
// Block b (tokens [bm, bm+m)) feeds two windows: the second half of entry b
// (window positions m..2m-1) and the first half of entry b+1 (positions
// 0..m-1).  With a reference r per dimension, a token's weight in either
// window factors as
//     exp(z + b_p - M) = 2^(z*log2e - r) * 2^((b_p - bmax)*log2e) * const,
// so each element needs one exp2, shared by both windows, times a
// per-position factor beta_p <= 1 precomputed once (in registers).  The
// constant cancels in the normalisation as long as both halves of an entry
// use the same r.  r moves only when a block maximum leaves [r - kBand,
// r + kBand] (log2 units); then the carried half is rescaled.  So weights
// stay in (2^-kBand-ish, 2^kBand] without a per-window maximum, and the
// result equals the exact softmax up to rounding.
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
  // carried first half (for the next entry) and the shared reference
  float cS[DPL], cA[DPL], ref[DPL];
  bool have_ref = false;
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
    // block maximum of z (log2 units) and the reference update
    float bmx[DPL];
#pragma unroll
    for (int d = 0; d < DPL; ++d) {
      float v = zc[0][d];
#pragma unroll
      for (int t = 1; t < M; ++t) v = fmaxf(v, zc[t][d]);
      bmx[d] = v * L2E;
    }
    bool move = !have_ref;
    if (have_ref) {
#pragma unroll
      for (int d = 0; d < DPL; ++d) move |= (bmx[d] > ref[d] + kBand) || (bmx[d] < ref[d] - kBand);
    }
    if (__any(move)) {
      // rescale the carried half to the new reference (exactly)
#pragma unroll
      for (int d = 0; d < DPL; ++d) {
        const float nr = next_ref(ref[d], bmx[d], have_ref);
        if (have_ref) {
          const float f = __builtin_amdgcn_exp2f(ref[d] - nr);
          cS[d] *= f;
          cA[d] *= f;
        }
        ref[d] = nr;
      }
      have_ref = true;
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
        const float u = __builtin_amdgcn_exp2f(fmaf(zc[t][d], L2E, -ref[d]));
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
        const float S = first ? sB[d] : cS[d] + sB[d];
        const float A = first ? aB[d] : cA[d] + aB[d];
        o[d] = A * __builtin_amdgcn_rcpf(S);
      }
      // rows outside [e0, e1) fall past the buffer record and are dropped
      const uint32_t off = (b >= e0 && b < e1) ? (uint32_t)((b - e0) * ld_out + d0) * sizeof(T)
                                               : 0xffffffffu;
      BufStoreN<T, DPL>::store(orsrc, off, o);
    }
#pragma unroll
    for (int d = 0; d < DPL; ++d) { cS[d] = sA[d]; cA[d] = aA[d]; }
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
