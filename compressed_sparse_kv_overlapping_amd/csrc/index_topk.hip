// Indexer scoring and top-k selection for gfx950.
//
// Method: "Frontier Techniques: NTK RoPE, CSA+HCA, QAT, MTP" 2.1 (entries
// scored cheaply by the indexer, the top 1024 kept per query) and "DeepSeek
// V4 comprimeix el context", section "CSA: buscar primer i atendre despres"
// (a light indexer scores every compressed entry and keeps the most relevant
// ones).  Score s[b][i] = scale * dot(q_idx[b], key[i]) over 64 dims; the
// selection is the first k visible entries in the order (score descending,
// index ascending).
//
// Selection without storing the B x N score matrix:
//  1. score pass (MFMA): scores are reduced to the maximum of every group of
//     GS consecutive entries.  The k-th largest group maximum is a score that
//     at least k entries reach, so it is a lower bound of the k-th best score.
//  2. threshold: per query, radix select of the k-th largest group maximum.
//  3. collect pass (MFMA again): every visible entry scoring at least the
//     threshold is appended to the query's candidate list (typically ~1.2 k
//     candidates for unstructured scores).
//  4. final: per query, exact radix select over (score key, ~index) 64-bit
//     composite keys of the candidates; the chosen indices are written in
//     ascending order (candidates are kept in entry-range order and sorted
//     only within each range).  If the candidate list overflowed (e.g. massive
//     score ties), the query is resolved by a self-contained streaming radix
//     select over all its entries instead.
#include <float.h>

#include <chrono>
#include <mutex>
#include <random>
#include <type_traits>

#include "common.hpp"
#include "fp4.hpp"
#include "kernels.hpp"

namespace cskv {

constexpr int kI = 64;
constexpr int kCap = 8192;           // candidate capacity per query
constexpr int kMaxK = 4096;
constexpr int kMaxGroups = 16384;

struct IdxArgs {
  const void* q;              // [B][64]
  const void* keys;           // [N][64] (+ b * key_bstride elements)
  const uint8_t* qsc;         // MXFP4 only: E8M0 scales [B][2]
  const uint8_t* ksc;         // MXFP4 only: E8M0 scales [N][2] (+ b * key_bstride / 32)
  const int64_t* q_pos;       // NULL at decode
  int64_t key_bstride;
  int B, N, k, m, GS, G, qpb, tiles_per_wave;
  int gs_shift;               // GS = 2^gs_shift
  float scale;
  uint32_t* gmax;             // [B][G]
  uint32_t* thr;              // [B]
  uint32_t* cnt;              // [B][chunks] candidates found per (query, chunk)
  uint64_t* cand;             // [B][chunks][region] candidate regions
  int32_t* out;               // [B][k]
  int chunks, region;         // score-pass chunks; slots per (query, chunk)
  int csize;                  // entries per chunk: chunk c holds entries [c csize, (c+1) csize)
  uint32_t cmagic;            // floor((2^32 - 1) / csize)
  float* sraw;                // per-sequence keys: raw scores [B][Np] kept between the passes, or NULL
  int64_t np;                 // row pitch of sraw (N rounded up to 16)
};

__device__ __forceinline__ int n_visible(const IdxArgs& a, int b) {
  if (!a.q_pos) return a.N;
  const int64_t v = (a.q_pos[b] + 1) / a.m;                 // entries with (i+1)m <= pos+1
  return (int)(v < 0 ? 0 : (v > a.N ? a.N : v));
}

template <class T> struct KeyFrag;
template <> struct KeyFrag<bf16_t> { static constexpr int bytes = 2; };
template <> struct KeyFrag<float> { static constexpr int bytes = 4; };
template <> struct KeyFrag<e4m3_t> { static constexpr int bytes = 1; };

// MXFP4 rows (OCP Microscaling v1.0; the format named for the indexer's QK
// path in "Frontier Techniques: NTK RoPE, CSA+HCA, QAT, MTP", QAT): 64 E2M1
// codes in 32 bytes, element 2j in the low nibble of byte j, and two E8M0
// scales per row (elements 0..31, 32..63) in a separate byte array.
struct fp4x2_t { uint8_t u; };
// MXFP4 on 16x16 tiles: the two halves f[0], f[1] of a lane's 16 codes (8
// bytes: dims 16 g .. 16 g + 15 of its row, g = l / 16) and the E8M0 byte of
// their block (g / 2), as the scaled MFMA takes it
template <> struct Frag<fp4x2_t> { uint32_t v; uint32_t s; };

// Bytes of a 64-element row, and the fragment type the MFMA consumes.
template <class T> struct Elem {
  static constexpr int kRowBytes = 64 * (int)sizeof(T);
  using QF = Frag<T>;
};
template <> struct Elem<fp4x2_t> {
  static constexpr int kRowBytes = 32;
  using QF = Frag<fp4x2_t>;
};

// Key fragments as the MFMA takes them.
template <class T>
__device__ __forceinline__ void key_decode(typename Elem<T>::QF* d, const Frag<T>* k) {
  d[0] = k[0];
  d[1] = k[1];
}

// S += keys . queries^T for one 16 x 16 tile over the 64 dims.  bf16, fp8,
// fp32: two MFMAs, k-step ks taking dims 32 ks + 8 g .. + 7 in lane group g.
// MXFP4: one v_mfma_scale 16x16x128 with E2M1 operands, lane group g
// supplying its 16 codes of block g / 2 in K slots 0..15 of its 32 (the
// other 16 zero) and that block's E8M0 scale, so each scale covers only its
// own block's elements; the products are exact, as with every format here.
template <class T>
__device__ __forceinline__ void score16(f32x4& S, const typename Elem<T>::QF* k,
                                        const typename Elem<T>::QF* q) {
  mma16(S, k[0], q[0]);
  mma16(S, k[1], q[1]);
}
template <>
__device__ __forceinline__ void score16<fp4x2_t>(f32x4& S, const Frag<fp4x2_t>* k,
                                                 const Frag<fp4x2_t>* q) {
  const v8i32_t a = {(int)k[0].v, (int)k[1].v, 0, 0, 0, 0, 0, 0};
  const v8i32_t b = {(int)q[0].v, (int)q[1].v, 0, 0, 0, 0, 0, 0};
  S = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, S, 4, 4, 0, (int)k[0].s, 0, (int)q[0].s);
}

// Both k-step fragments (dims 0..31 and 32..63, slots 8g..8g+7) of row r,
// from global memory: kb = the rows' first byte, sb = their scales (MXFP4).
template <class T>
__device__ __forceinline__ void key_frags(Frag<T>* f, const char* kb, const uint8_t* sb, int64_t r,
                                          int g) {
  const T* p = reinterpret_cast<const T*>(kb + r * Elem<T>::kRowBytes);
  frag_load(f[0], p + 8 * g);
  frag_load(f[1], p + 32 + 8 * g);
}
template <>
__device__ __forceinline__ void key_frags<fp4x2_t>(Frag<fp4x2_t>* f, const char* kb, const uint8_t* sb,
                                                   int64_t r, int g) {
  const uint2 w = *reinterpret_cast<const uint2*>(kb + r * 32 + 8 * g);
  f[0].v = w.x;
  f[1].v = w.y;
  f[0].s = f[1].s = sb[2 * r + (g >> 1)];
}

// The block scale of row r for fragments whose codes came from LDS.
template <class T>
__device__ __forceinline__ void key_scales(Frag<T>* f, const uint8_t* sb, int64_t r, int g) {}
template <>
__device__ __forceinline__ void key_scales<fp4x2_t>(Frag<fp4x2_t>* f, const uint8_t* sb, int64_t r,
                                                    int g) {
  f[0].s = f[1].s = sb[2 * r + (g >> 1)];
}

// Query row r's fragments, decoded once per kernel.
template <class T>
__device__ __forceinline__ void query_frags(typename Elem<T>::QF* f, const IdxArgs& a, int64_t r,
                                            int g) {
  Frag<T> raw[2];
  key_frags<T>(raw, reinterpret_cast<const char*>(a.q), a.qsc, r, g);
  key_decode<T>(f, raw);
}

// Maximum of two scores in one instruction: the median of (a, b, +inf),
// which skips the quieting of signalling NaNs that the compiler puts before
// an IEEE-mode maximum (scores of finite inputs are never NaN).  pinf holds
// +inf in a register the compiler cannot see into, so that it keeps the
// median instead of turning it back into a maximum.
__device__ __forceinline__ float max_raw(float a, float b, float pinf) {
  return __builtin_amdgcn_fmed3f(a, b, pinf);
}

// Neighbours of a float in the total order of finite values (zero steps to
// the smallest denormal of the other side).
__device__ __forceinline__ float next_up(float x) {
  if (x != x || x == INFINITY) return x;
  if (x == 0.f) return __uint_as_float(1u);
  const uint32_t u = __float_as_uint(x);
  return __uint_as_float(x > 0.f ? u + 1u : u - 1u);
}
__device__ __forceinline__ float next_down(float x) { return -next_up(-x); }

// The smallest raw dot product S with fl(S * scale) >= t (scale > 0): the
// product is monotone in S, so S >= this bound exactly when the scaled score
// reaches t.  Starts from fl(t / scale), within an ulp or two of the bound;
// if the search does not settle (only for absurd scales) every score
// qualifies, which is still exact (the final select sorts it out).
__device__ float raw_threshold(float t, float scale) {
  if (t == -INFINITY) return -INFINITY;
  float s = t / scale;
  for (int i = 0; i < 8 && !(s * scale >= t); ++i) s = next_up(s);
  for (int i = 0; i < 8; ++i) {
    const float p = next_down(s);
    if (p * scale >= t) s = p; else break;
  }
  const bool ok = s * scale >= t && !(next_down(s) * scale >= t);
  return ok ? s : -INFINITY;
}

// Key rows staged in LDS for the many-query score passes: 16 KB stages of
// whole 64-dim rows (kRow bytes each), the 16-byte chunks of row r stored at
// chunk c ^ swz(r).  16 consecutive rows then put a lane group's fragment
// reads on distinct banks (rows per 256 bytes: 4 fp8, 2 bf16, 1 fp32).
template <class T> struct KeyTiles {
  static constexpr int kRow = Elem<T>::kRowBytes;
  static constexpr int kChunks = kRow / 16;
  static constexpr int kRowsPer256 = 256 / kRow;
  static constexpr int kStage = 16384;
  static constexpr int kTiles = kStage / (16 * kRow);        // 16-row tiles per stage
  static __device__ __forceinline__ int swz(int r) { return (r / kRowsPer256) % kChunks; }
  // byte offset of the fragment of k-step ks, lane group g, in a row
  static __device__ __forceinline__ int frag_off(int ks, int g) {
    if constexpr (std::is_same<T, fp4x2_t>::value) return 8 * g + 4 * ks;   // the lane's 8 code bytes
    return (32 * ks + 8 * g) * kRow / 64;
  }
  // the 8-element fragment at byte offset off of a staged row
  static __device__ __forceinline__ void load(Frag<T>& f, const char* row, int off, int sw);
};
template <> __device__ __forceinline__ void KeyTiles<fp4x2_t>::load(Frag<fp4x2_t>& f, const char* row,
                                                                    int off, int sw) {
  f.v = *reinterpret_cast<const uint32_t*>(row + 16 * ((off >> 4) ^ sw) + (off & 15));
}
template <> __device__ __forceinline__ void KeyTiles<e4m3_t>::load(Frag<e4m3_t>& f, const char* row,
                                                                   int off, int sw) {
  f.v = *reinterpret_cast<const uint64_t*>(row + 16 * ((off >> 4) ^ sw) + (off & 15));
}
template <> __device__ __forceinline__ void KeyTiles<bf16_t>::load(Frag<bf16_t>& f, const char* row,
                                                                   int off, int sw) {
  f.v = *reinterpret_cast<const u32x4*>(row + 16 * ((off >> 4) ^ sw));
}
template <> __device__ __forceinline__ void KeyTiles<float>::load(Frag<float>& f, const char* row,
                                                                  int off, int sw) {
  const u32x4 a = *reinterpret_cast<const u32x4*>(row + 16 * ((off >> 4) ^ sw));
  const u32x4 b = *reinterpret_cast<const u32x4*>(row + 16 * (((off >> 4) + 1) ^ sw));
  f.v[0] = __uint_as_float(a.x); f.v[1] = __uint_as_float(a.y);
  f.v[2] = __uint_as_float(a.z); f.v[3] = __uint_as_float(a.w);
  f.v[4] = __uint_as_float(b.x); f.v[5] = __uint_as_float(b.y);
  f.v[6] = __uint_as_float(b.z); f.v[7] = __uint_as_float(b.w);
}

// MODE 0: group maxima.  MODE 1: collect candidates >= threshold into this
// chunk's region of each query (counted in LDS, no global atomics).
//
// WQ = 1: the block's waves share 16*NQB queries and split the chunk's
// entries.  WQ = 4: each wave owns 16*NQB queries of its own and all four
// stream the same entry tiles (read once from L2 per block, then hit in L1),
// which divides the key traffic of many-query launches by four.
//
// Tiles that every query of the wave sees entirely take a fast epilogue: a
// running maximum (MODE 0), or one comparison of the raw MFMA score against
// the threshold divided by the scale (MODE 1).
template <class T, int NQB, int MODE, int WQ>
__global__ __launch_bounds__(256) void idx_score_kernel(IdxArgs a) {
  __shared__ uint32_t lcnt[WQ * 16 * NQB];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int qw = WQ == 4 ? wave : 0;                         // this wave's query set
  if (MODE == 1) {
    if (threadIdx.x < WQ * 16 * NQB) lcnt[threadIdx.x] = 0;
    __syncthreads();
  }
  const int col = lane & 15, g = lane >> 4;
  const int q0 = blockIdx.y * a.qpb + qw * 16 * NQB;
  // per-sequence keys: key_bstride elements per query (a multiple of 64)
  const int64_t krow0 = (int64_t)q0 * (a.key_bstride / kI);
  const char* kbase = reinterpret_cast<const char*>(a.keys) + krow0 * Elem<T>::kRowBytes;
  const uint8_t* sbase = a.ksc ? a.ksc + 2 * krow0 : nullptr;

  // this lane's queries (one per 16-column block) and their query fragments
  typename Elem<T>::QF qf[NQB][2];
  int qb[NQB], nvis[NQB];
  float tscore[NQB], traw[NQB];
  int blk_vis = 0, min_vis = 0x7fffffff;
#pragma unroll
  for (int j = 0; j < NQB; ++j) {
    const int c = 16 * j + col;
    const bool ok = (WQ == 4 || c < a.qpb) && q0 + c < a.B;
    qb[j] = ok ? q0 + c : -1;
    nvis[j] = ok ? n_visible(a, q0 + c) : 0;
    blk_vis = max(blk_vis, nvis[j]);
    min_vis = min(min_vis, ok ? nvis[j] : 0x7fffffff);
    if (ok) {
      query_frags<T>(qf[j], a, q0 + c, g);
    } else {
      typename Elem<T>::QF z{};
      qf[j][0] = z;
      qf[j][1] = z;
    }
    tscore[j] = -INFINITY;                                       // threshold 0: take all
    if (MODE == 1 && ok && a.thr[q0 + c] != 0u) tscore[j] = key_score(a.thr[q0 + c]);
    traw[j] = MODE == 1 && ok ? raw_threshold(tscore[j], a.scale) : INFINITY;   // absent: none
  }
  // the largest visible prefix over the wave's queries bounds the tiles; up
  // to the smallest one every tile is fully visible
  for (int off = 32; off >= 1; off >>= 1) {
    blk_vis = max(blk_vis, __shfl_xor(blk_vis, off, 64));
    min_vis = min(min_vis, __shfl_xor(min_vis, off, 64));
  }

  // group maxima are written for every group (0 when nothing is visible);
  // candidates are only looked for in the visible prefix
  const int e_w0 = (WQ == 4 ? blockIdx.x : blockIdx.x * 4 + wave) * a.tiles_per_wave * 16;
  const int e_w1 = min(e_w0 + a.tiles_per_wave * 16, MODE == 0 ? a.G * a.GS : blk_vis);
  float pinf = INFINITY;
  asm volatile("" : "+v"(pinf));
  // running group maximum of this lane's query per 16-column block (a lane's
  // four entries of a tile always lie in one group: GS >= 4)
  float gm[NQB];
#pragma unroll
  for (int j = 0; j < NQB; ++j) gm[j] = -INFINITY;

  // group maxima (GS >= 16): lane g keeps the maximum of group 4n + g, and
  // every fourth group (or the range's last) the lanes write the 16 bytes of
  // up to four consecutive groups of their query at once
  float held[NQB];
  const int grp_first = e_w0 >> a.gs_shift, grp_last = (e_w1 - 1) >> a.gs_shift;
  auto tile = [&](const int et, const Frag<T>* kf) {
   if (et < blk_vis) {                                         // skip invisible tiles
    typename Elem<T>::QF kd[2];
    key_decode<T>(kd, kf);
    f32x4 S[NQB];
#pragma unroll
    for (int j = 0; j < NQB; ++j) {
      S[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      score16<T>(S[j], kd, qf[j]);
    }
    // S[j][i]: query qb[j], entry et + 4g + i
    if (MODE == 0 && NQB == 1 && a.sraw && qb[0] >= 0)         // one query per block
      *reinterpret_cast<f32x4*>(a.sraw + (int64_t)qb[0] * a.np + et + 4 * g) = S[0];
    if (et + 16 <= min_vis) {
      if (MODE == 0) {
#pragma unroll
        for (int j = 0; j < NQB; ++j)
          gm[j] = max_raw(max_raw(gm[j], max_raw(S[j][0], S[j][1], pinf), pinf),
                          max_raw(S[j][2], S[j][3], pinf), pinf);
      } else {
        bool hit = false;
#pragma unroll
        for (int j = 0; j < NQB; ++j)
          hit |= max_raw(max_raw(S[j][0], S[j][1], pinf), max_raw(S[j][2], S[j][3], pinf), pinf) >= traw[j];
        if (__any(hit)) {
#pragma unroll
          for (int j = 0; j < NQB; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              if (S[j][i] >= traw[j] && qb[j] >= 0) {
                const int e = et + 4 * g + i;
                const float s = S[j][i] * a.scale;
                const uint32_t slot = atomicAdd(&lcnt[qw * 16 * NQB + 16 * j + col], 1u);
                if (slot < (uint32_t)a.region)
                  a.cand[((int64_t)qb[j] * a.chunks + blockIdx.x) * a.region + slot] =
                      ((uint64_t)score_key(s) << 32) | (uint64_t)(0xffffffffu - (uint32_t)e);
              }
            }
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < NQB; ++j) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = et + 4 * g + i;
          const bool vis = e < nvis[j];
          if (MODE == 0) {
            gm[j] = fmaxf(gm[j], vis ? S[j][i] : -INFINITY);
          } else if (vis && S[j][i] >= traw[j]) {
            const float s = S[j][i] * a.scale;
            const uint32_t slot = atomicAdd(&lcnt[qw * 16 * NQB + 16 * j + col], 1u);
            if (slot < (uint32_t)a.region)
              a.cand[((int64_t)qb[j] * a.chunks + blockIdx.x) * a.region + slot] =
                  ((uint64_t)score_key(s) << 32) | (uint64_t)(0xffffffffu - (uint32_t)e);
          }
        }
      }
    }
   }
    if (MODE == 0) {
      // group boundaries coincide with tile boundaries for GS >= 16
      const int GS = a.GS;
      if (GS <= 8 || ((et + 16) & (GS - 1)) == 0) {
#pragma unroll
        for (int j = 0; j < NQB; ++j) {
          float v = gm[j];
          if (GS <= 8) {
            int grp;
            bool writer;
            if (GS == 4) {
              grp = (et + 4 * g) / 4;
              writer = true;
            } else {
              v = fmaxf(v, shfl_xor(v, 16));
              grp = (et + 8 * (g >> 1)) / 8;
              writer = (g & 1) == 0;
            }
            if (writer && qb[j] >= 0 && grp < a.G)
              a.gmax[(int64_t)qb[j] * a.G + grp] = (v == -INFINITY) ? 0u : score_key(v * a.scale);
          } else {
            v = fmaxf(v, shfl_xor(v, 16));
            v = fmaxf(v, shfl_xor(v, 32));
            const int grp = et >> a.gs_shift;
            if (g == (grp & 3)) held[j] = v;
            if ((grp & 3) == 3 || grp == grp_last) {
              const int gw = (grp & ~3) + g;                   // this lane's group
              if (gw >= grp_first && gw <= grp && qb[j] >= 0 && gw < a.G)
                a.gmax[(int64_t)qb[j] * a.G + gw] =
                    (held[j] == -INFINITY) ? 0u : score_key(held[j] * a.scale);
            }
          }
          gm[j] = -INFINITY;
        }
      }
    }
  };

  if constexpr (WQ == 1) {
    // key fragments of the next PF - 1 tiles are in flight while a tile is
    // computed (register ring, the loop unrolled by PF so slots are fixed)
    constexpr int PF = 4;
    Frag<T> kr[PF][2];
    auto load_tile = [&](const int et, Frag<T>* kf) {
      const int er = et + col;                                 // A row of this lane
      if (et < e_w1 && et < blk_vis && er < a.N) {
        key_frags<T>(kf, kbase, sbase, er, g);
      } else {
        Frag<T> z{};
        kf[0] = z;
        kf[1] = z;
      }
    };
#pragma unroll
    for (int p = 0; p < PF - 1; ++p) load_tile(e_w0 + 16 * p, kr[p]);
    for (int et = e_w0; et < e_w1; et += 16 * PF) {
      load_tile(et + 48, kr[3]);
      tile(et, kr[0]);
      if (et + 16 >= e_w1) break;
      load_tile(et + 64, kr[0]);
      tile(et + 16, kr[1]);
      if (et + 32 >= e_w1) break;
      load_tile(et + 80, kr[1]);
      tile(et + 32, kr[2]);
      if (et + 48 >= e_w1) break;
      load_tile(et + 96, kr[2]);
      tile(et + 48, kr[3]);
    }
  } else {
    // The block's key rows pass through LDS in stages of 16 KB, copied by
    // all four waves straight from global memory while the previous stage is
    // computed.  Rows are kept whole with their 16-byte chunks XOR-swizzled
    // by row, so the fragment reads of 16 consecutive rows hit distinct banks.
    using KT = KeyTiles<T>;
    __shared__ __attribute__((aligned(16))) char kst[2][KT::kStage];
    __shared__ int sh_end[4];
    if (lane == 0) sh_end[wave] = e_w1;
    __syncthreads();
    const int e_b1 = max(max(sh_end[0], sh_end[1]), max(sh_end[2], sh_end[3]));
    const int nst = e_b1 > e_w0 ? (e_b1 - e_w0 + 16 * KT::kTiles - 1) / (16 * KT::kTiles) : 0;
    const char* keys = reinterpret_cast<const char*>(a.keys);
    auto issue = [&](const int st) {
      char* buf = kst[st & 1];
#pragma unroll
      for (int n = 0; n < KT::kStage / 4096; ++n) {
        const int pos = (n * 4 + wave) * 1024 + lane * 16;     // byte in the stage
        const int r = pos / KT::kRow, c = (pos % KT::kRow) / 16;
        int row = e_w0 + st * 16 * KT::kTiles + r;
        row = row < a.N ? row : a.N - 1;
        const char* src = keys + (int64_t)row * KT::kRow + 16 * (c ^ KT::swz(r));
        dma16(src, (unsigned)__builtin_amdgcn_readfirstlane(lds_offset(buf + (n * 4 + wave) * 1024)));
      }
    };
    if (nst > 0) issue(0);
    const int swz = KT::swz(col);
    for (int st = 0; st < nst; ++st) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();                                         // stage st landed; st - 1 read
      if (st + 1 < nst) issue(st + 1);
      const char* buf = kst[st & 1];
      // fragments of the next tile are read from LDS while a tile computes
      Frag<T> kf[2][2];
      auto frags = [&](const int t, Frag<T>* f) {
        const char* rowp = buf + (t * 16 + col) * KT::kRow;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) KT::load(f[ks], rowp, KT::frag_off(ks, g), swz);
        const int row = e_w0 + (st * KT::kTiles + t) * 16 + col;   // as staged (clamped)
        key_scales<T>(f, sbase, row < a.N ? row : a.N - 1, g);
      };
      frags(0, kf[0]);
      static_assert(KT::kTiles % 2 == 0, "tiles per stage come in pairs");
      for (int t = 0; t < KT::kTiles; t += 2) {
        const int et = e_w0 + (st * KT::kTiles + t) * 16;
        if (et >= e_w1) break;
        frags(t + 1, kf[1]);
        tile(et, kf[0]);
        if (et + 16 >= e_w1) break;
        if (t + 2 < KT::kTiles) frags(t + 2, kf[0]);
        tile(et + 16, kf[1]);
      }
    }
  }
  if (MODE == 1) {
    __syncthreads();
    if (threadIdx.x < WQ * 16 * NQB) {
      const int c = threadIdx.x;
      const int q = blockIdx.y * a.qpb + c;
      if ((WQ == 4 || c < a.qpb) && q < a.B) a.cnt[(int64_t)q * a.chunks + blockIdx.x] = lcnt[c];
    }
  }
}

// ---------------------------------------------------------------------------
// Many-query score passes on 32x32 MFMA tiles.
//
// A block of four waves takes one chunk of entries and 4 x 32 NQB queries:
// wave w owns queries q0 + 32 NQB w + 32 j + (l % 32), j < NQB, and the four
// waves read the same key rows, staged in LDS in 16 KB stages exactly as in
// the kernel above.  A tile is 32 entries:
//   S[j] = keys (32 x 64) . queries_j^T (64 x 32)
// one MFMA over all 64 dims for fp8 and MXFP4 (v_mfma_scale 32x32x64 with
// the f8f6f4 operand formats: each lane supplies 32 consecutive dims of its
// row, dims 32 (l / 32) .. + 31, i.e. one MX block, with that block's E8M0
// scale; for fp8 the scales are 2^0), four 32x32x16 MFMAs for bf16.  Lane l
// then holds query l % 32 and the 16 entries 8 (i / 4) + 4 (l / 32) + i % 4
// of the tile, so a lane reduces 16 scores of one query.
//
// MODE 0: group maxima (GS >= 32, groups aligned to tiles): a running
// maximum over the lane's scores (v_max3), the two lane halves joined with a
// permlane swap at the end of a group; lane half g keeps group 2n + g and
// writes it every second group.  MODE 1: candidates >= the threshold: the
// lane's 16 scores of a tile are reduced to their maximum the same way, and
// a lane whose maximum reaches its query's threshold (a few lanes per tile)
// queues the 16 scores as one block in LDS; when the queue fills, and at the
// end, every lane takes one block and appends the entries that qualify to
// the per-(query, chunk) candidate regions.  The hit test costs no more than
// the group maximum, and per-score work is left to the few queued blocks.
template <class T> struct Tile32;
template <> struct Tile32<e4m3_t> {
  using BFrag = v8i32_t;
  static constexpr int kFmt = 0;
};
template <> struct Tile32<fp4x2_t> {
  using BFrag = v8i32_t;
  static constexpr int kFmt = 4;
};
template <> struct Tile32<bf16_t> {
  struct BFrag { u32x4 s[4]; };
  static constexpr int kFmt = 1;
};

// The lane's operand of row `row` of a 64-dim row image at p (global memory
// or a staged row whose 16-byte chunk c sits at chunk c ^ sw).
template <class T>
__device__ __forceinline__ void tile32_frag(typename Tile32<T>::BFrag& f, const char* row, int sw,
                                            int g);
template <>
__device__ __forceinline__ void tile32_frag<e4m3_t>(v8i32_t& f, const char* row, int sw, int g) {
  const u32x4 a = *reinterpret_cast<const u32x4*>(row + 16 * ((2 * g) ^ sw));
  const u32x4 b = *reinterpret_cast<const u32x4*>(row + 16 * ((2 * g + 1) ^ sw));
  f = v8i32_t{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}
template <>
__device__ __forceinline__ void tile32_frag<fp4x2_t>(v8i32_t& f, const char* row, int sw, int g) {
  const u32x4 a = *reinterpret_cast<const u32x4*>(row + 16 * (g ^ sw));
  f = v8i32_t{(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
}
template <>
__device__ __forceinline__ void tile32_frag<bf16_t>(Tile32<bf16_t>::BFrag& f, const char* row, int sw,
                                                    int g) {
#pragma unroll
  for (int s = 0; s < 4; ++s) f.s[s] = *reinterpret_cast<const u32x4*>(row + 16 * ((2 * s + g) ^ sw));
}

// S = A . B over the 64 dims (sa, sb: E8M0 scales of the lanes' blocks, MXFP4 only)
template <class T>
__device__ __forceinline__ f32x16 tile32_mma(const typename Tile32<T>::BFrag& a,
                                             const typename Tile32<T>::BFrag& b, int sa, int sb) {
  const f32x16 z = {};
  if constexpr (Tile32<T>::kFmt == 0) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, z, 0, 0, 0, 127, 0, 127);
  } else {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, z, 4, 4, 0, sa, 0, sb);
  }
}
template <>
__device__ __forceinline__ f32x16 tile32_mma<bf16_t>(const Tile32<bf16_t>::BFrag& a,
                                                     const Tile32<bf16_t>::BFrag& b, int, int) {
  f32x16 c = {};
#pragma unroll
  for (int s = 0; s < 4; ++s)
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a.s[s]),
                                                __builtin_bit_cast(bf16x8, b.s[s]), c, 0, 0, 0);
  return c;
}

constexpr int kQB = 64;                      // per-wave queue of lane blocks (one tile's worst case)

template <class T, int NQB, int MODE, int GSL>
__global__ __launch_bounds__(256) void idx_score32_kernel(IdxArgs a) {
  using KT = KeyTiles<T>;
  using F = typename Tile32<T>::BFrag;
  constexpr int kT32 = KT::kStage / (32 * KT::kRow);          // 32-row tiles per stage
  constexpr int QW = 32 * NQB;                                // queries per wave
  constexpr int QB = MODE == 1 ? kQB : 1;
  __shared__ __attribute__((aligned(16))) char kst[2][KT::kStage];
  __shared__ uint32_t lcnt[4 * QW];
  // MODE 1: queued lane blocks (a lane's 16 scores of one tile), their
  // first entry and query slot, and the raw threshold of each query slot
  __shared__ __attribute__((aligned(16))) float qs[4][QB][16];
  __shared__ uint32_t qm[4][QB];
  __shared__ float qt[4][MODE == 1 ? QW : 1];
  __shared__ int sh_end[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hq = lane & 31, g = lane >> 5;
  const int qw0 = blockIdx.y * a.qpb + wave * QW;              // this wave's first query
  if (MODE == 1) {
    for (int i = threadIdx.x; i < 4 * QW; i += 256) lcnt[i] = 0;
  }

  // the lane's queries: operands, visible counts, thresholds
  F qf[NQB];
  int qb[NQB], nvis[NQB], qsc[NQB];
  float traw[NQB];
  int blk_vis = 0, min_vis = 0x7fffffff;
#pragma unroll
  for (int j = 0; j < NQB; ++j) {
    const int q = qw0 + 32 * j + hq;
    const bool ok = q < a.B;
    qb[j] = ok ? q : -1;
    nvis[j] = ok ? n_visible(a, q) : 0;
    blk_vis = max(blk_vis, nvis[j]);
    min_vis = min(min_vis, ok ? nvis[j] : 0x7fffffff);
    const char* qrow = reinterpret_cast<const char*>(a.q) + (int64_t)(ok ? q : 0) * KT::kRow;
    tile32_frag<T>(qf[j], qrow, 0, g);
    if (!ok) qf[j] = F{};
    qsc[j] = 127;
    if constexpr (Tile32<T>::kFmt == 4) qsc[j] = ok ? a.qsc[(int64_t)q * 2 + g] : 127;
    float tscore = -INFINITY;                                // threshold 0: take all
    if (MODE == 1 && ok && a.thr[q] != 0u) tscore = key_score(a.thr[q]);
    // rows past the visible count score -inf and never qualify, also when
    // every visible entry does (scores are finite)
    traw[j] = MODE == 1 && ok ? fmaxf(raw_threshold(tscore, a.scale), -FLT_MAX) : INFINITY;
    if (MODE == 1) qt[wave][32 * j + hq] = traw[j];
  }
  for (int off = 32; off >= 1; off >>= 1) {
    blk_vis = max(blk_vis, __shfl_xor(blk_vis, off, 64));
    min_vis = min(min_vis, __shfl_xor(min_vis, off, 64));
  }
  blk_vis = __builtin_amdgcn_readfirstlane(blk_vis);
  min_vis = __builtin_amdgcn_readfirstlane(min_vis);

  const int e_w0 = blockIdx.x * a.tiles_per_wave * 16;
  const int e_w1 = min(e_w0 + a.tiles_per_wave * 16, MODE == 0 ? a.G * a.GS : blk_vis);
  if (lane == 0) sh_end[wave] = e_w1;
  __syncthreads();
  const int e_b1 = max(max(sh_end[0], sh_end[1]), max(sh_end[2], sh_end[3]));
  const int nst = e_b1 > e_w0 ? (e_b1 - e_w0 + 32 * kT32 - 1) / (32 * kT32) : 0;
  const char* keys = reinterpret_cast<const char*>(a.keys);
  const int64_t krow0 = 0;                                   // shared keys (per-sequence keys take the other kernels)
  const uint8_t* ksc = a.ksc;

  // MODE 0 state: running maxima; a stage's closed groups wait in registers
  // (lane half g keeps groups 2n + g) and are stored early in the next
  // stage, so that the stage's wait for its key tiles does not wait for them
  constexpr int GS = 1 << GSL;
  constexpr int kPend = MODE == 0 ? 16 * kT32 / GS : 1;      // groups per stage per lane half
  static_assert(MODE == 1 || (GS >= 32 && 32 * kT32 % (2 * GS) == 0), "groups of whole tiles, even per stage");
  float gm[NQB], pend[NQB][kPend];
#pragma unroll
  for (int j = 0; j < NQB; ++j) {
    gm[j] = -INFINITY;
#pragma unroll
    for (int s = 0; s < kPend; ++s) pend[j][s] = -INFINITY;
  }
  const int g_end = e_w1 >> GSL;                             // groups [.., g_end) are computed
  auto store_stage = [&](const int st) {
    const int g0 = (e_w0 + st * 32 * kT32) >> GSL;
#pragma unroll
    for (int s = 0; s < kPend; ++s) {
      const int gw = g0 + 2 * s + g;
#pragma unroll
      for (int j = 0; j < NQB; ++j)
        if (qb[j] >= 0 && gw < g_end)
          a.gmax[(int64_t)qb[j] * a.G + gw] = pend[j][s] == -INFINITY ? 0u : score_key(pend[j][s] * a.scale);
    }
  };
  // MODE 1 state: the wave's queue fill (uniform)
  int qn = 0;
  auto flush = [&]() {
    // a lane a block: the registers at or above the query's threshold, then
    // one candidate slot per such register
    for (int b0 = 0; b0 < qn; b0 += 64) {
      const int i = b0 + lane;
      if (i < qn) {
        const uint32_t meta = qm[wave][i];
        const int ql = (int)(meta >> 24), e0 = (int)(meta & 0xffffffu);
        const float t = qt[wave][ql];
        uint32_t hits = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(&qs[wave][i][4 * c]);
          hits |= ((uint32_t)(v.x >= t) | ((uint32_t)(v.y >= t) << 1) | ((uint32_t)(v.z >= t) << 2) |
                   ((uint32_t)(v.w >= t) << 3)) << (4 * c);
        }
        uint64_t* dst = a.cand + ((int64_t)(qw0 + ql) * a.chunks + blockIdx.x) * a.region;
        while (hits) {
          const int r = __builtin_ctz(hits);
          hits &= hits - 1u;
          const int e = e0 + 8 * (r >> 2) + (r & 3);
          const uint32_t key = score_key(qs[wave][i][r] * a.scale);
          const uint32_t slot = atomicAdd(&lcnt[wave * QW + ql], 1u);
          if (slot < (uint32_t)a.region) dst[slot] = ((uint64_t)key << 32) | (uint64_t)(0xffffffffu - (uint32_t)e);
        }
      }
    }
    qn = 0;
  };

  // one 32-entry tile: both column blocks' products first, so that they
  // overlap; rows past a query's visible count masked (register i holds row
  // et + 4 g + 8 (i / 4) + i % 4); then the lane's maximum: the group maximum
  // (MODE 0) or the hit test (MODE 1: a lane whose 16 scores reach the
  // threshold queues all of them; one reservation per tile, few lanes
  // qualify)
  auto tile = [&](const int et, const F& kf, const int ksa) {
    if (et >= blk_vis) return;
    f32x16 SS[NQB];
#pragma unroll
    for (int j = 0; j < NQB; ++j) SS[j] = tile32_mma<T>(kf, qf[j], ksa, qsc[j]);
    if (et + 32 > min_vis) {
#pragma unroll
      for (int j = 0; j < NQB; ++j) {
        const int lim = nvis[j] - et - 4 * g;
#pragma unroll
        for (int i = 0; i < 16; ++i) SS[j][i] = 8 * (i >> 2) + (i & 3) < lim ? SS[j][i] : -INFINITY;
      }
    }
#pragma unroll
    for (int j = 0; j < NQB; ++j) {
      const f32x16& S = SS[j];
      float m = MODE == 0 ? gm[j] : -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; i += 2) m = fmaxf(fmaxf(m, S[i]), S[i + 1]);
      if (MODE == 0) {
        gm[j] = m;
      } else {
        const bool hit = m >= traw[j];
        const uint64_t hm = __ballot(hit);
        if (hm) {
          const int n = __builtin_popcountll(hm);
          if (qn + n > kQB) flush();
          if (hit) {
            const int pos = qn + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(hm >> 32),
                                                                __builtin_amdgcn_mbcnt_lo((uint32_t)hm, 0u));
            f32x4* d = reinterpret_cast<f32x4*>(&qs[wave][pos][0]);
            d[0] = f32x4{S[0], S[1], S[2], S[3]};
            d[1] = f32x4{S[4], S[5], S[6], S[7]};
            d[2] = f32x4{S[8], S[9], S[10], S[11]};
            d[3] = f32x4{S[12], S[13], S[14], S[15]};
            qm[wave][pos] = (uint32_t)(et + 4 * g) | ((uint32_t)(32 * j + hq) << 24);
          }
          qn += n;
        }
      }
    }
  };
  // MODE 0: tile t of a stage closes group (32 t) / GS of the stage when
  // 32 (t + 1) is a multiple of GS: the two lane halves are joined
  auto close = [&](const int t) {
    if (MODE == 0 && (32 * (t + 1)) % GS == 0) {
      const int lg = (32 * t) / GS;
#pragma unroll
      for (int j = 0; j < NQB; ++j) {
        const float v = max_xor32(gm[j]);                     // both lane halves' rows
        if ((lg & 1) == g) pend[j][lg >> 1] = v;
        gm[j] = -INFINITY;
      }
    }
  };

  auto issue = [&](const int st) {
    char* buf = kst[st & 1];
#pragma unroll
    for (int n = 0; n < KT::kStage / 4096; ++n) {
      const int pos = (n * 4 + wave) * 1024 + lane * 16;     // byte in the stage
      const int r = pos / KT::kRow, c = (pos % KT::kRow) / 16;
      int row = e_w0 + st * 32 * kT32 + r;
      row = row < a.N ? row : a.N - 1;
      const char* src = keys + (krow0 + row) * KT::kRow + 16 * (c ^ KT::swz(r));
      dma16(src, (unsigned)__builtin_amdgcn_readfirstlane(lds_offset(buf + (n * 4 + wave) * 1024)));
    }
  };
  if (nst > 0) issue(0);
  for (int st = 0; st < nst; ++st) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();                                         // stage st landed; st - 1 read
    if (st + 1 < nst) issue(st + 1);
    if (MODE == 0 && st > 0) store_stage(st - 1);
    // the lane's row in a staged tile is 32 t + l % 32, whose swizzle does
    // not depend on t
    const char* buf = kst[st & 1] + hq * KT::kRow;
    const int sw = KT::swz(hq);
    // MXFP4: the key block scales, fetched one tile ahead
    int ksa_next = 127;
    if constexpr (Tile32<T>::kFmt == 4) ksa_next = ksc[(krow0 + min(e_w0 + st * kT32 * 32 + hq, a.N - 1)) * 2 + g];
    // the next tile's key operand is read from LDS while a tile computes
    F kf, kn;
    tile32_frag<T>(kn, buf, sw, g);
#pragma unroll
    for (int t = 0; t < kT32; ++t) {
      const int et = e_w0 + (st * kT32 + t) * 32;
      if (et >= e_w1) break;
      kf = kn;
      if (t + 1 < kT32) tile32_frag<T>(kn, buf + (t + 1) * 32 * KT::kRow, sw, g);
      const int ksa = ksa_next;
      if constexpr (Tile32<T>::kFmt == 4)
        ksa_next = ksc[(krow0 + min(et + 32 + hq, a.N - 1)) * 2 + g];
      tile(et, kf, ksa);
      close(t);
    }
  }
  if (MODE == 0 && nst > 0) store_stage(nst - 1);
  if (MODE == 1) {
    flush();
    __syncthreads();
    for (int c = threadIdx.x; c < 4 * QW; c += 256) {
      const int q = blockIdx.y * a.qpb + c;
      if (q < a.B) a.cnt[(int64_t)q * a.chunks + blockIdx.x] = lcnt[c];
    }
  }
}

// Collect pass from kept scores (per-sequence keys): the same candidates as
// the MODE 1 score pass, read from the raw scores the group-maximum pass
// stored instead of recomputed from the keys, so every key is read once.
// Block (chunk c, query b) covers the entries the score pass gave chunk c.
__global__ __launch_bounds__(256) void idx_collect_kept_kernel(IdxArgs a) {
  __shared__ uint32_t lcnt;
  const int b = blockIdx.y, c = blockIdx.x;
  if (threadIdx.x == 0) lcnt = 0;
  __syncthreads();
  const int e0 = c * a.tiles_per_wave * 16 * 4;
  const int e1 = min(e0 + a.tiles_per_wave * 16 * 4, n_visible(a, b));
  const float tscore = a.thr[b] != 0u ? key_score(a.thr[b]) : -INFINITY;
  const float traw = raw_threshold(tscore, a.scale);
  const float* sr = a.sraw + (int64_t)b * a.np;
  for (int e = e0 + threadIdx.x; e < e1; e += 256) {
    const float v = sr[e];
    if (v >= traw) {
      const uint32_t slot = atomicAdd(&lcnt, 1u);
      if (slot < (uint32_t)a.region)
        a.cand[((int64_t)b * a.chunks + c) * a.region + slot] =
            ((uint64_t)score_key(v * a.scale) << 32) | (uint64_t)(0xffffffffu - (uint32_t)e);
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) a.cnt[(int64_t)b * a.chunks + c] = lcnt;
}

// ------------------------------------------------- block-wide radix helpers

// Exclusive prefix sum over the block (256 threads): wave scans, then the
// wave totals.  *total receives the block sum.  part[] holds 4 values.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t x, uint32_t* part, uint32_t* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t incl = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  if (lane == 63) part[w] = incl;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    const uint32_t p = part[i];
    base += i < w ? p : 0u;
    tot += p;
  }
  __syncthreads();                                           // part[] free again
  *total = tot;
  return base + incl - x;
}

// Bin of hist[nbins] (nbins a multiple of NT, NT threads) that holds the
// kk-th largest counted key: thread t owns the t-th group of nbins/NT bins
// from the top.  *sh_digit gets the bin, *sh_above the keys in higher bins.
template <int NT>
__device__ void find_kth_bin(const uint32_t* hist, int nbins, uint32_t kk, uint32_t* sh_digit,
                             uint32_t* sh_above, uint32_t* part) {
  const int t = threadIdx.x;
  const int per = nbins / NT;
  uint32_t local = 0;
  for (int i = 0; i < per; ++i) local += hist[nbins - 1 - (t * per + i)];
  uint32_t tot;
  const uint32_t before = block_excl_scan<NT>(local, part, &tot);
  if (before < kk && kk <= before + local) {
    uint32_t cum = before;
    for (int i = 0; i < per; ++i) {
      const int bin = nbins - 1 - (t * per + i);
      if (cum + hist[bin] >= kk) {
        *sh_digit = (uint32_t)bin;
        *sh_above = cum;
        break;
      }
      cum += hist[bin];
    }
  }
  __syncthreads();
}

// Block min and max of the valid keys (NT threads; part[] holds NT / 32
// values).
template <int NT>
__device__ __forceinline__ void block_minmax(uint32_t mn, uint32_t mx, uint32_t* part, uint32_t* out_mn,
                                             uint32_t* out_mx) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, off, 64));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, 64));
  }
  if (lane == 0) { part[w] = mn; part[NT / 64 + w] = mx; }
  __syncthreads();
  mn = part[0];
  mx = part[NT / 64];
#pragma unroll
  for (int i = 1; i < NT / 64; ++i) {
    mn = min(mn, part[i]);
    mx = max(mx, part[NT / 64 + i]);
  }
  __syncthreads();
  *out_mn = mn;
  *out_mx = mx;
}

// Block sum of the counts and min and max of the keys in one exchange (NT
// threads; part[] holds 3 NT / 64 values).
template <int NT>
__device__ __forceinline__ void block_count_minmax(uint32_t n, uint32_t mn, uint32_t mx, uint32_t* part,
                                                   uint32_t* out_n, uint32_t* out_mn, uint32_t* out_mx) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    n += (uint32_t)__shfl_xor((int)n, off, 64);
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, off, 64));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, 64));
  }
  if (lane == 0) { part[w] = n; part[NW + w] = mn; part[2 * NW + w] = mx; }
  __syncthreads();
  n = part[0];
  mn = part[NW];
  mx = part[2 * NW];
#pragma unroll
  for (int i = 1; i < NW; ++i) {
    n += part[i];
    mn = min(mn, part[NW + i]);
    mx = max(mx, part[2 * NW + i]);
  }
  __syncthreads();
  *out_n = n;
  *out_mn = mn;
  *out_mx = mx;
}

// kk-th largest (1-based) of the 32-bit keys that key_at(i) yields as valid,
// i in [0, n), given their min lo and max hi.  Every pass spreads the
// remaining range over 2^BB bins of equal width, so keys crowded into a few
// high bits still fall into distinct bins (few colliding LDS atomics) and a
// range of 2^r takes ceil(r / BB) passes.  *above_out: valid keys greater
// than the result.
template <int BB, int NT, class KeyAt>
__device__ uint32_t block_kth_largest(KeyAt key_at, int n, uint32_t kk, uint32_t lo, uint32_t hi,
                                      uint32_t* hist, uint32_t* part, uint32_t* sh_digit,
                                      uint32_t* sh_above, uint32_t* above_out) {
  uint32_t above_total = 0;
  for (;;) {
    const uint32_t range = hi - lo;
    if (range == 0) break;
    const int bits = 32 - __clz((int)range);              // range < 2^bits
    const int shift = bits > BB ? bits - BB : 0;
    for (int i = threadIdx.x; i < (1 << BB); i += NT) hist[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += NT) {
      uint32_t key;
      if (key_at(i, key) && key >= lo && key <= hi) atomicAdd(&hist[(key - lo) >> shift], 1u);
    }
    __syncthreads();
    find_kth_bin<NT>(hist, 1 << BB, kk, sh_digit, sh_above, part);
    const uint32_t bin = *sh_digit;
    kk -= *sh_above;
    above_total += *sh_above;
    __syncthreads();
    lo += bin << shift;
    const uint32_t top = lo + ((1u << shift) - 1u);
    hi = top < hi ? top : hi;
    if (shift == 0) break;
  }
  *above_out = above_total;
  return lo;
}

// The k-th largest of the G group maxima of each query (0 if fewer than k
// non-empty groups or fewer than k visible entries): at least k groups, hence
// k entries, reach it, and no coarse bin lets extra entries in (one group
// whose maximum is near zero, e.g. at the causal edge, would otherwise widen
// the key range and with it the bins).  Up to 16 maxima a thread stay in
// registers (else they are re-read from L2): one histogram of 4096 bins over
// their key range, then the few maxima in the bin that holds the k-th are
// ranked directly (a crowded bin takes further histogram passes).
// Loads and stores of data that other blocks of the same launch write or
// read (COH): system-scope accesses, which write through and read past the
// XCD's L2, so that no cache write-back or invalidation is needed between
// the phases of the fused decode kernel.  Plain accesses otherwise.
template <bool COH, class U>
__device__ __forceinline__ U ld_c(const U* p) {
  if constexpr (COH) return __hip_atomic_load(const_cast<U*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  else return *p;
}
template <bool COH, class U>
__device__ __forceinline__ void st_c(U* p, U v) {
  if constexpr (COH) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  else *p = v;
}

// The threshold of query b, by a block of NT threads.  LDS: hist[4096],
// part[3 NT / 64] and four words, each its own __shared__ object in the
// caller (inlined there, so the compiler sees that they do not overlap).
template <int NT, bool COH = false>
__device__ __forceinline__ void threshold_query(const IdxArgs& a, const int b, uint32_t* hist, uint32_t* part,
                                                uint32_t& sh_digit, uint32_t& sh_above, uint32_t& sh_n,
                                                uint32_t& sh_tau) {
  constexpr int kPer = 16;
  constexpr uint32_t kRank = 128;                            // bin members ranked directly
  const int t = threadIdx.x;
  const uint32_t* gm = a.gmax + (int64_t)b * a.G;
  const bool held = a.G <= kPer * NT;
  uint32_t v[kPer];
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int i = t + r * NT;
    v[r] = held && i < a.G ? ld_c<COH>(gm + i) : 0u;
  }
  // the histogram below, cleared while the maxima load
  for (int i = t; i < 4096; i += NT) hist[i] = 0;
  if (t == 0) sh_n = 0;
  auto each = [&](auto&& f) {                                // every non-empty group's maximum
    if (held) {
#pragma unroll
      for (int r = 0; r < kPer; ++r)
        if (v[r] != 0u) f(v[r]);
    } else {
      for (int i = t; i < a.G; i += NT) {
        const uint32_t x = ld_c<COH>(gm + i);
        if (x != 0u) f(x);
      }
    }
  };
  uint32_t ne = 0, mn = 0xffffffffu, mx = 0u;
  each([&](uint32_t x) { ++ne; mn = min(mn, x); mx = max(mx, x); });
  // (its block barriers also order the cleared histogram before its use)
  uint32_t nonempty, lo, hi;
  block_count_minmax<NT>(ne, mn, mx, part, &nonempty, &lo, &hi);
  const int nv = n_visible(a, b);
  if (nv <= a.k || nonempty < (uint32_t)a.k) {
    if (t == 0) st_c<COH>(a.thr + b, 0u);
    return;
  }
  const uint32_t range = hi - lo;
  const int bits = range ? 32 - __clz((int)range) : 0;     // range < 2^bits
  const int shift = bits > 12 ? bits - 12 : 0;
  each([&](uint32_t x) { atomicAdd(&hist[(x - lo) >> shift], 1u); });
  __syncthreads();
  find_kth_bin<NT>(hist, 4096, (uint32_t)a.k, &sh_digit, &sh_above, part);
  const uint32_t bin = sh_digit, kk = (uint32_t)a.k - sh_above, nbin = hist[bin];
  __syncthreads();                                           // hist is read; it holds the members next
  if (nbin <= kRank) {
    each([&](uint32_t x) {
      if (((x - lo) >> shift) == bin) hist[atomicAdd(&sh_n, 1u)] = x;
    });
    __syncthreads();
    // the member with fewer than kk larger ones and at least kk at or above
    for (uint32_t m = t; m < nbin; m += NT) {
      const uint32_t x = hist[m];
      uint32_t gt = 0, ge = 0;
      for (uint32_t j = 0; j < nbin; ++j) {
        gt += hist[j] > x;
        ge += hist[j] >= x;
      }
      if (gt < kk && kk <= ge) sh_tau = x;                   // equal maxima write the same value
    }
    __syncthreads();
    if (t == 0) st_c<COH>(a.thr + b, sh_tau);
    return;
  }
  const uint32_t blo = lo + (bin << shift), span = (1u << shift) - 1u;
  const uint32_t bhi = hi - blo > span ? blo + span : hi;
  uint32_t above;
  const uint32_t tau = block_kth_largest<12, NT>(
      [&](int i, uint32_t& key) { key = ld_c<COH>(gm + i); return key != 0u; }, a.G, kk, blo, bhi, hist, part,
      &sh_digit, &sh_above, &above);
  if (t == 0) st_c<COH>(a.thr + b, tau);
}

template <int NT>
__global__ __launch_bounds__(NT) void idx_threshold_kernel(IdxArgs a) {
  __shared__ uint32_t hist[4096], part[3 * NT / 64];
  __shared__ uint32_t sh_digit, sh_above, sh_n, sh_tau;
  threshold_query<NT>(a, blockIdx.x, hist, part, sh_digit, sh_above, sh_n, sh_tau);
}

// ----------------------------------------------------------------- final


// 64-bit composite of the scored entry e: score key high, ~e low (so that
// larger composite = higher score, then lower index).
__device__ __forceinline__ uint64_t composite(uint32_t key, int e) {
  return ((uint64_t)key << 32) | (uint64_t)(0xffffffffu - (uint32_t)e);
}

template <class T>
__device__ __forceinline__ float dot64(const T* qrow, const T* krow);
// Raw score of query b and entry e (key rows of query b when per sequence).
template <class T>
__device__ __forceinline__ float entry_dot(const IdxArgs& a, int b, int e) {
  const T* kb = reinterpret_cast<const T*>(a.keys) + (int64_t)b * a.key_bstride;
  return dot64<T>(reinterpret_cast<const T*>(a.q) + (int64_t)b * kI, kb + (int64_t)e * kI);
}
template <> __device__ __forceinline__ float dot64<float>(const float* q, const float* k) {
  float s = 0.f;
  for (int r = 0; r < kI; ++r) s = fmaf(q[r], k[r], s);
  return s;
}
template <> __device__ __forceinline__ float dot64<bf16_t>(const bf16_t* q, const bf16_t* k) {
  float s = 0.f;
  for (int r = 0; r < kI; ++r)
    s = fmaf(__uint_as_float((uint32_t)q[r].u << 16), __uint_as_float((uint32_t)k[r].u << 16), s);
  return s;
}
template <> __device__ __forceinline__ float dot64<e4m3_t>(const e4m3_t* q, const e4m3_t* k) {
  float s = 0.f;
  for (int r = 0; r < kI; ++r)
    s = fmaf(__builtin_amdgcn_cvt_f32_fp8((int)q[r].u, 0), __builtin_amdgcn_cvt_f32_fp8((int)k[r].u, 0), s);
  return s;
}
template <>
__device__ __forceinline__ float entry_dot<fp4x2_t>(const IdxArgs& a, int b, int e) {
  const int64_t kr = (int64_t)b * (a.key_bstride / kI) + e;
  const uint32_t* q = reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(a.q) + (int64_t)b * 32);
  const uint32_t* k = reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(a.keys) + kr * 32);
  float s = 0.f;
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    const float sq = __uint_as_float(e8m0_f32_bits(a.qsc[(int64_t)b * 2 + blk]));
    const float sk = __uint_as_float(e8m0_f32_bits(a.ksc[kr * 2 + blk]));
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t qw = q[4 * blk + w], kw = k[4 * blk + w];
#define CSKV_FP4_PAIR(SEL)                                                          \
      {                                                                             \
        const hw_f32x2_t qv = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(qw, sq, SEL);    \
        const hw_f32x2_t kv = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(kw, sk, SEL);    \
        s = fmaf(qv[0], kv[0], s);                                                  \
        s = fmaf(qv[1], kv[1], s);                                                  \
      }
      CSKV_FP4_PAIR(0) CSKV_FP4_PAIR(1) CSKV_FP4_PAIR(2) CSKV_FP4_PAIR(3)
#undef CSKV_FP4_PAIR
    }
  }
  return s;
}

// Exact selection for one query.  Candidates are either the collected list
// (in LDS) or, on overflow, every visible entry with its score recomputed.
//
// Collected list: the candidate regions are gathered in chunk order, i.e. in
// ascending entry ranges.  The k-th largest composite is found with one
// histogram of the score words over 2048 bins of their range; the few
// candidates in the bin that holds it are ranked exactly by composite (a
// crowded bin falls back to further passes).  The selected candidates,
// compacted in list order, are then in ascending order of chunk; each is
// written at the start of its chunk's run plus its rank by index within that
// run, so the output is ascending without a global sort.
constexpr int kMaxChunks = 2048;
constexpr int kFinalBB = 11;                 // histogram of 2^11 bins
constexpr int kMem = 512;                    // bin members ranked exactly
//
// CAP: candidate capacity in LDS (2048 for k <= 1024, so that five blocks fit
// on a compute unit; 8192 otherwise).  A query with more candidates takes
// the streaming path, with the same result.
// candidates (list) or, on overflow, the k <= CAP / 2 selected indices
template <int CAP> union FinalCands { uint64_t cand[CAP]; int32_t sel[CAP / 2]; };
// the histogram, then the members of the k-th bin, then where each chunk's
// selected candidates start and end in the compacted list
union FinalHist { uint32_t hist[1 << kFinalBB]; uint64_t mem[kMem]; uint16_t seg[2][kMaxChunks]; };

// The selection of query b, by a block of NT threads.  LDS: the candidate
// and histogram unions, coff[kMaxChunks + 1] (list offset of each chunk),
// part[NT / 32] and five words, separate __shared__ objects in the callers
// that can have them (inlined there, so the compiler sees that they do not
// overlap).
template <class T, int NT, int CAP, bool COH = false>
__device__ __forceinline__ void final_query(const IdxArgs& a, const int b, FinalCands<CAP>& cs, FinalHist& hs,
                                            uint16_t* coff, uint32_t* part, uint32_t& sh_digit,
                                            uint32_t& sh_above, uint32_t& sh_nsel, uint32_t& sh_over,
                                            uint64_t& sh_thr) {
  static_assert(CAP <= kCap && CAP / 2 <= kMaxK, "capacity");
  uint64_t* cand = cs.cand;
  int32_t* sel = cs.sel;
  uint32_t* hist = hs.hist;
  const int t = threadIdx.x;
  const int nv = n_visible(a, b);
  int32_t* out = a.out + (int64_t)b * a.k;
  if (nv <= a.k) {
    for (int j = t; j < a.k; j += NT) out[j] = j < nv ? j : -1;
    return;
  }
  // gather: thread t owns chunks [c0, c1); a full region or more than kCap
  // candidates in total means overflow
  if (t == 0) sh_over = 0;
  const bool listed = a.chunks <= kMaxChunks;               // else: streaming path
  const int cpt = (a.chunks + NT - 1) / NT;
  const int c0 = listed ? min(a.chunks, t * cpt) : 0, c1 = listed ? min(a.chunks, c0 + cpt) : 0;
  uint32_t mine = 0;
  bool full = !listed;
  for (int c = c0; c < c1; ++c) {
    const uint32_t n = ld_c<COH>(a.cnt + (int64_t)b * a.chunks + c);
    full |= n > (uint32_t)a.region;
    mine += n > (uint32_t)a.region ? (uint32_t)a.region : n;
  }
  __syncthreads();
  if (full) sh_over = 1;
  uint32_t total;
  const uint32_t base = block_excl_scan<NT>(mine, part, &total);
  const bool overflow = sh_over != 0 || total > (uint32_t)CAP;
  // list slots of this thread (gather and output), and the chunk of p0
  const uint32_t per = (total + NT - 1) / NT;
  const uint32_t p0 = min(total, t * per), p1 = min(total, p0 + per);
  uint32_t mn = 0xffffffffu, mx = 0u;                        // score words of this thread's slots
  if (!overflow) {
    // chunk offsets in the list, then a copy spread over the whole block:
    // list slot j belongs to the last chunk whose offset is <= j
    uint32_t at = base;
    for (int c = c0; c < c1; ++c) {
      coff[c] = (uint16_t)at;
      const uint32_t n = ld_c<COH>(a.cnt + (int64_t)b * a.chunks + c);
      at += n > (uint32_t)a.region ? (uint32_t)a.region : n;
    }
    if (t == 0) coff[a.chunks] = (uint16_t)total;
    __syncthreads();
    // thread t copies list slots [p0, p1): the chunk of p0 by binary search,
    // then a walk (chunks are contiguous in the list), the loads issued
    // eight at a time
    if (p0 < p1) {
      int lo = 0, hi = a.chunks;                             // coff[lo] <= p0 < coff[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (coff[mid] <= p0) lo = mid; else hi = mid;
      }
      int c = lo;
      uint32_t cb = coff[c], ce = coff[c + 1];
      for (uint32_t p = p0; p < p1; p += 8) {
        uint64_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const uint32_t q = p + u;
          if (q < p1) {
            while (q >= ce) {
              ++c;
              cb = ce;
              ce = coff[c + 1];
            }
            v[u] = ld_c<COH>(a.cand + ((int64_t)b * a.chunks + c) * a.region + (q - cb));
          }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (p + u < p1) {
            cand[p + u] = v[u];
            mn = min(mn, (uint32_t)(v[u] >> 32));
            mx = max(mx, (uint32_t)(v[u] >> 32));
          }
      }
    }
    // the histogram of the selection below, cleared while the copies land
    for (int i = t; i < (1 << kFinalBB); i += NT) hist[i] = 0;
    if (t == 0) { sh_nsel = 0; sh_thr = 0; }
  }
  const int nc = overflow ? 0 : (int)total;

  // the k-th largest composite
  uint64_t prefix = 0;
  if (!overflow) {
    // the block barriers of the range reduction also order the copies and
    // the cleared histogram before their readers
    uint32_t lo, hi;
    block_minmax<NT>(mn, mx, part, &lo, &hi);
    const uint32_t range = hi - lo;
    const int bits = range ? 32 - __clz((int)range) : 0;   // range < 2^bits
    const int shift = bits > kFinalBB ? bits - kFinalBB : 0;
    for (int j = t; j < nc; j += NT)
      atomicAdd(&hist[((uint32_t)(cand[j] >> 32) - lo) >> shift], 1u);
    __syncthreads();
    find_kth_bin<NT>(hist, 1 << kFinalBB, (uint32_t)a.k, &sh_digit, &sh_above, part);
    const uint32_t bin = sh_digit, kk = (uint32_t)a.k - sh_above, nbin = hist[bin];
    __syncthreads();                                         // hist is read; mem reuses it
    if (nbin <= (uint32_t)kMem) {
      // the bin's members; the one with exactly kk - 1 larger members is
      // the k-th largest overall (composites are distinct)
      for (int j = t; j < nc; j += NT) {
        const uint64_t v = cand[j];
        if ((((uint32_t)(v >> 32) - lo) >> shift) == bin) hs.mem[atomicAdd(&sh_nsel, 1u)] = v;
      }
      __syncthreads();
      for (uint32_t i = t; i < nbin; i += NT) {
        const uint64_t v = hs.mem[i];
        uint32_t r = 0;
        for (uint32_t j = 0; j < nbin; ++j) r += hs.mem[j] > v;
        if (r == kk - 1) sh_thr = v;
      }
      __syncthreads();
      prefix = sh_thr;
    } else {
      // a crowded bin: the score word by further passes, then the index
      // word among the candidates tied on that score
      uint32_t above;
      const uint32_t th = block_kth_largest<kFinalBB, NT>(
          [&](int j, uint32_t& key) { key = (uint32_t)(cand[j] >> 32); return true; }, nc,
          (uint32_t)a.k, lo, hi, hist, part, &sh_digit, &sh_above, &above);
      const uint32_t kt = (uint32_t)a.k - above;             // to take among score th
      mn = 0xffffffffu;
      mx = 0u;
      for (int j = t; j < nc; j += NT) {
        const uint64_t v = cand[j];
        if ((uint32_t)(v >> 32) == th) {
          mn = min(mn, (uint32_t)v);
          mx = max(mx, (uint32_t)v);
        }
      }
      block_minmax<NT>(mn, mx, part, &lo, &hi);
      const uint32_t tl = block_kth_largest<kFinalBB, NT>(
          [&](int j, uint32_t& key) {
            const uint64_t v = cand[j];
            key = (uint32_t)v;
            return (uint32_t)(v >> 32) == th;
          },
          nc, kt, lo, hi, hist, part, &sh_digit, &sh_above, &above);
      prefix = ((uint64_t)th << 32) | tl;
      __syncthreads();                                       // hist is read; the placement reuses it
    }
  } else {
    // radix select over the recomputed composites, digits of 11, 11 and 10
    // bits per 32-bit word
    uint64_t mask = 0;
    uint32_t kk = (uint32_t)a.k;
    bool done = false;
    for (int p = 0; p < 6 && !done; ++p) {
      const int bits = (p % 3 == 2) ? 10 : 11;
      const int shift = 64 - 32 * (p / 3) - (p % 3 == 0 ? 11 : (p % 3 == 1 ? 22 : 32));
      const uint32_t nb = 1u << bits;
      for (int i = t; i < (int)nb; i += NT) hist[i] = 0;
      __syncthreads();
      for (int e = t; e < nv; e += NT) {
        const float s = entry_dot<T>(a, b, e) * a.scale;
        const uint64_t v = composite(score_key(s), e);
        if ((v & mask) == prefix) atomicAdd(&hist[(uint32_t)(v >> shift) & (nb - 1)], 1u);
      }
      __syncthreads();
      find_kth_bin<NT>(hist, (int)nb, kk, &sh_digit, &sh_above, part);
      kk -= sh_above;
      const uint32_t bucket = hist[sh_digit];
      prefix |= (uint64_t)sh_digit << shift;
      mask |= (uint64_t)(nb - 1) << shift;
      done = bucket == kk;               // every key in the bucket is selected
      __syncthreads();
    }
  }
  // threshold: the k-th largest composite (on overflow the lowest one of
  // the final bucket); composites are distinct, so exactly k reach it
  const uint64_t thr = prefix;
  if (!overflow) {
    // placement.  The list is in chunk order and chunks are ascending entry
    // ranges, so the output (ascending indices) is the selected candidates in
    // list order with each chunk's run sorted by index.  The selected low
    // words are compacted in list order (each thread its own run of slots,
    // one block scan), each chunk's run is delimited, and every selected
    // candidate goes to its run's start plus the number of the run's members
    // with a smaller index (a larger low word).
    constexpr int U = CAP / NT;                              // list slots a thread holds at most
    uint32_t los[U];
    uint32_t selm = 0, nmine = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t j = p0 + u;
      const uint64_t v = cand[j < (uint32_t)CAP ? j : CAP - 1];
      const bool s = j < p1 && v >= thr;
      los[u] = (uint32_t)v;
      selm |= (uint32_t)s << u;
      nmine += s;
    }
    uint32_t nsel;
    uint32_t at = block_excl_scan<NT>(nmine, part, &nsel);
    // the scan's barriers order every read of the list before these writes
    uint32_t* run = reinterpret_cast<uint32_t*>(cand);
#pragma unroll
    for (int u = 0; u < U; ++u)
      if ((selm >> u) & 1u) run[at++] = los[u];
    __syncthreads();
    const uint32_t cs_ = (uint32_t)a.csize;
    auto chunk_of = [&](const uint32_t lo) {
      const uint32_t e = 0xffffffffu - lo;
      uint32_t c = __umulhi(e, a.cmagic);                    // floor(e / csize) or one less
      return c + (e - c * cs_ >= cs_ ? 1u : 0u);
    };
    // G list positions a thread at a time, their loads issued together;
    // nl <= k <= CAP / 2 keeps every read below inside the list's storage
    // (2 CAP words)
    constexpr int G = CAP / 2 / NT < 4 ? CAP / 2 / NT : 4;
    static_assert(G >= 1, "a position per thread");
    const uint32_t nl = min(nsel, (uint32_t)a.k);
    uint16_t* first = hs.seg[0];
    uint16_t* last = hs.seg[1];
    for (uint32_t i0 = t; i0 < nl; i0 += G * NT) {
      uint32_t w0[G], w1[G], w2[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const uint32_t i = i0 + g * NT < nl ? i0 + g * NT : 0u;
        w0[g] = run[i > 0 ? i - 1 : 0];
        w1[g] = run[i];
        w2[g] = run[i + 1];
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const uint32_t i = i0 + g * NT;
        if (i < nl) {
          const uint32_t c = chunk_of(w1[g]);
          if (i == 0 || chunk_of(w0[g]) != c) first[c] = (uint16_t)i;
          if (i + 1 == nl || chunk_of(w2[g]) != c) last[c] = (uint16_t)(i + 1);
        }
      }
    }
    __syncthreads();
    // rank within the run, eight words at a time; the words past a run (at
    // most seven beyond the longest of the G) are not counted
    for (uint32_t i0 = t; i0 < nl; i0 += G * NT) {
      uint32_t lo[G], L[G], n[G], r[G];
      uint32_t span = 0;
#pragma unroll
      for (int g = 0; g < G; ++g) lo[g] = run[i0 + g * NT < nl ? i0 + g * NT : 0u];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const uint32_t c = chunk_of(lo[g]);
        L[g] = first[c];
        n[g] = i0 + g * NT < nl ? last[c] - L[g] : 0u;
        r[g] = 0;
        span = max(span, n[g]);
      }
      for (uint32_t j = 0; j < span; j += 8) {
        uint32_t w[G][8];
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int u = 0; u < 8; ++u) w[g][u] = run[L[g] + j + u];
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int u = 0; u < 8; ++u) r[g] += (j + u < n[g] && w[g][u] > lo[g]) ? 1u : 0u;
      }
#pragma unroll
      for (int g = 0; g < G; ++g)
        if (i0 + g * NT < nl && L[g] + r[g] < (uint32_t)a.k) out[L[g] + r[g]] = (int32_t)(0xffffffffu - lo[g]);
    }
    for (int j = (int)nsel + t; j < a.k; j += NT) out[j] = -1;
    return;
  }
  // overflow: collect the selected indices by streaming, then sort them
  if (t == 0) sh_nsel = 0;
  __syncthreads();
  for (int e = t; e < nv; e += NT) {
    const float s = entry_dot<T>(a, b, e) * a.scale;
    if (composite(score_key(s), e) >= thr) {
      const uint32_t at = atomicAdd(&sh_nsel, 1u);
      if (at < (uint32_t)(CAP / 2)) sel[at] = e;
    }
  }
  __syncthreads();
  int n2 = 1;
  while (n2 < a.k) n2 <<= 1;
  for (int j = a.k + t; j < n2; j += NT) sel[j] = 0x7fffffff;
  __syncthreads();
  for (int size = 2; size <= n2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = t; i < n2 / 2; i += NT) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const int32_t x = sel[lo], y = sel[hi];
        if ((x > y) == up) { sel[lo] = y; sel[hi] = x; }
      }
      __syncthreads();
    }
  }
  for (int j = t; j < a.k; j += NT) out[j] = sel[j];
}

template <class T, int NT, int CAP>
__global__ __launch_bounds__(NT) void idx_final_kernel(IdxArgs a) {
  __shared__ FinalCands<CAP> cs;
  __shared__ FinalHist hs;
  __shared__ uint16_t coff[kMaxChunks + 1];
  __shared__ uint32_t part[NT / 32];
  __shared__ uint32_t sh_digit, sh_above, sh_nsel, sh_over;
  __shared__ uint64_t sh_thr;
  final_query<T, NT, CAP>(a, blockIdx.x, cs, hs, coff, part, sh_digit, sh_above, sh_nsel, sh_over, sh_thr);
}

// ------------------------------------------------------------ decode, fused
//
// The decode selection (up to 32 queries over one shared, fully visible key
// set) in a single launch: the four steps above run as phases of one kernel,
// with one block of 1024 threads resident on every compute unit.  Block c
// owns the C keys [c C, c C + C):
//  A. scores its keys for every query (the same 16x16 MFMA steps as the
//     score passes, so the same raw scores), keeps the raw scores in LDS and
//     writes its groups' maxima;
//  B. (blocks b < B, once every block is past A) the threshold of query b,
//     as idx_threshold_kernel;
//  C. (once every threshold is out) appends its candidates, read from LDS
//     rather than recomputed, to the per-(query, block) regions;
//  D. (blocks b < B, once every block is past C) the exact selection of
//     query b, as idx_final_kernel.
// The result is that of the four launches.  The phase words live in the
// workspace, which holds whatever its last user left: each launch passes a
// 64-bit tag of its own and phase i publishes tag + i, which stale contents
// match with probability about 2^-64.  Waits are bounded, so a grid that is
// not resident ends with the error word set instead of hanging.
constexpr int kDecThreads = 1024;
constexpr int kDecPad = 4;                                   // row pad of the score array (floats)
constexpr int kDecScores = 32 * (1024 + kDecPad);            // 128.5 KB of raw scores
constexpr uint32_t kDecSpin = 1u << 24;                      // polls of a wait (tens of seconds) before giving up

constexpr int kDecMaxBlocks = 256;                           // flag words: four a lane of one wave
constexpr int kDecFlagStride = 8;                            // 64-bit flag words 64 bytes apart

struct DecodeBar {
  uint64_t err, pad0[7];
  uint64_t a[kDecMaxBlocks * kDecFlagStride];                // block c's phase A is done
  uint64_t b[32 * kDecFlagStride];                           // query q's threshold is out
  uint64_t c[kDecMaxBlocks * kDecFlagStride];                // block c's phase C is done
};

// The blocks exchange data through system-scope accesses (ld_c / st_c with
// COH), which write through and read past the L2s, so no cache write-back or
// invalidation is needed between phases; only each wave's stores must have
// completed (a block barrier alone does not wait for them).  A block then
// publishes a phase's value (the launch's tag + phase number) in its own
// word (no shared counter: same-address atomics from every block
// serialise), and a block that needs the phase waits for exactly the words
// it depends on, polled by one wave, four a lane: a single memory round trip
// from the last publisher to the waiter.  Every wait is bounded: past the
// limit the error word is set and the block goes on.
__device__ __forceinline__ void dec_publish(uint64_t* word, uint64_t value) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) st_c<true>(word, value);
}
// words[i * kDecFlagStride] == value for every i < n (n <= 256)
__device__ __forceinline__ void dec_wait(DecodeBar* bar, const uint64_t* words, int n, uint64_t value) {
  if (threadIdx.x < 64) {
    const int f0 = 4 * threadIdx.x;
    uint32_t spins = 0;
    for (;;) {
      bool done = true;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (f0 + u < n) done &= ld_c<true>(&words[(f0 + u) * kDecFlagStride]) == value;
      if (__all(done)) break;
      __builtin_amdgcn_s_sleep(2);
      if (++spins == kDecSpin) {
        if (threadIdx.x == 0) st_c<true>(&bar->err, value);
        break;
      }
    }
  }
  __syncthreads();
}

// raw scores [16 NQB][C + kDecPad] (phases A to C), then phase D's lists
template <int CAP> union DecodeScores {
  float sc[kDecScores];
  struct { FinalCands<CAP> cs; FinalHist hs; uint16_t coff[kMaxChunks + 1]; } fin;
};

// C keys a block (a multiple of 256 and of 16 GS: whole 16-key tiles for
// each of the 16 waves, and whole groups in each wave's keys); bar: the
// phase words; tag: the launch's tag.
template <class T, int NQB, int CAP>
__global__ __launch_bounds__(kDecThreads) void idx_decode_kernel(IdxArgs a, int C, DecodeBar* bar,
                                                                uint64_t tag) {
  __shared__ DecodeScores<CAP> u;
  __shared__ uint32_t thist[4096], part[3 * kDecThreads / 64];  // phases B and D
  __shared__ uint32_t sh_digit, sh_above, sh_n, sh_tau, sh_over;
  __shared__ uint64_t sh_thr;
  __shared__ uint32_t lcnt[32];                              // phase C: candidates per query
  __shared__ float traw[32];                                 // phase C: raw thresholds
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int blk = blockIdx.x;
  const int P = C + kDecPad;                                 // score row pitch
  const int64_t c0 = (int64_t)blk * C;
  float* sc = u.sc;

  // A. raw scores of the block's keys: wave w takes keys c0 + w C/16 + ...
  {
    typename Elem<T>::QF qf[NQB][2];
#pragma unroll
    for (int j = 0; j < NQB; ++j) {
      const int q = 16 * j + col;
      if (q < a.B) {
        query_frags<T>(qf[j], a, q, g);
      } else {
        typename Elem<T>::QF z{};
        qf[j][0] = z;
        qf[j][1] = z;
      }
    }
    const char* kb = reinterpret_cast<const char*>(a.keys);
    const int per = C / 16;                                  // keys per wave (a multiple of 16 and of GS)
    float pinf = INFINITY;
    asm volatile("" : "+v"(pinf));
    const int GS = a.GS;
    // group maxima as the tiles go: a lane's four scores of a tile lie in one
    // group (GS >= 4); GS = 8 joins lane groups g and g ^ 1, GS >= 16 all
    // four, and larger groups run across the wave's consecutive tiles
    float gm[NQB];
#pragma unroll
    for (int j = 0; j < NQB; ++j) gm[j] = -INFINITY;
    auto put_max = [&](const int q, const int64_t key, const float m) {
      const int64_t gi = key >> a.gs_shift;
      if (q < a.B && gi < a.G)
        st_c<true>(a.gmax + (int64_t)q * a.G + gi, (m == -INFINITY) ? 0u : score_key(m * a.scale));
    };
    // tiles in flight a wave (fp32 fragments are twice the registers)
    constexpr int TF = sizeof(T) == 4 ? 2 : 4;
    for (int t0 = 0; t0 < per; t0 += 16 * TF) {
      Frag<T> kf[TF][2];
#pragma unroll
      for (int u = 0; u < TF; ++u) {
        const int64_t er = c0 + wave * per + t0 + 16 * u + col;
        if (t0 + 16 * u < per && er < a.N) {
          key_frags<T>(kf[u], kb, a.ksc, er, g);
        } else {
          Frag<T> z{};
          kf[u][0] = z;
          kf[u][1] = z;
        }
      }
#pragma unroll
      for (int u = 0; u < TF; ++u) {
        const int el = wave * per + t0 + 16 * u;             // first key of the tile, in the block
        if (t0 + 16 * u < per) {
          typename Elem<T>::QF kd[2];
          key_decode<T>(kd, kf[u]);
#pragma unroll
          for (int j = 0; j < NQB; ++j) {
            f32x4 S = f32x4{0.f, 0.f, 0.f, 0.f};
            score16<T>(S, kd, qf[j]);
            // S[i]: query 16 j + col, key c0 + el + 4 g + i (-inf past N)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (c0 + el + 4 * g + i >= a.N) S[i] = -INFINITY;
            *reinterpret_cast<f32x4*>(sc + (16 * j + col) * P + el + 4 * g) = S;
            float m = max_raw(max_raw(S[0], S[1], pinf), max_raw(S[2], S[3], pinf), pinf);
            if (GS == 4) {
              put_max(16 * j + col, c0 + el + 4 * g, m);
            } else if (GS == 8) {
              m = max_raw(m, __shfl_xor(m, 16, 64), pinf);
              if ((g & 1) == 0) put_max(16 * j + col, c0 + el + 4 * g, m);
            } else {
              m = max_raw(m, __shfl_xor(m, 16, 64), pinf);
              m = max_raw(m, __shfl_xor(m, 32, 64), pinf);
              gm[j] = max_raw(gm[j], m, pinf);
              if (((el + 16) & (GS - 1)) == 0) {             // the tile closes a group
                if (g == 0) put_max(16 * j + col, c0 + el, gm[j]);
                gm[j] = -INFINITY;
              }
            }
          }
        }
      }
    }
  }
  dec_publish(&bar->a[blk * kDecFlagStride], tag + 1u);

  // B. thresholds: query q in block q, once every block's group maxima are out
  if (blk < a.B) {
    dec_wait(bar, bar->a, gridDim.x, tag + 1u);
    threshold_query<kDecThreads, true>(a, blk, thist, part, sh_digit, sh_above, sh_n, sh_tau);
    dec_publish(&bar->b[blk * kDecFlagStride], tag + 2u);
  }
  dec_wait(bar, bar->b, a.B, tag + 2u);

  // C. candidates >= the threshold, from the scores in LDS
  if (threadIdx.x < a.B) {
    const uint32_t th = ld_c<true>(a.thr + threadIdx.x);
    traw[threadIdx.x] = raw_threshold(th != 0u ? key_score(th) : -INFINITY, a.scale);
    lcnt[threadIdx.x] = 0u;
  }
  __syncthreads();
  {
    // each lane reads back the scores it wrote in phase A
    const int per = C / 16;
    for (int t = 0; t < per; t += 16) {
      const int el = wave * per + t;
#pragma unroll
      for (int j = 0; j < NQB; ++j) {
        const int q = 16 * j + col;
        if (q >= a.B) continue;
        const f32x4 S = *reinterpret_cast<const f32x4*>(sc + q * P + el + 4 * g);
        const float tr = traw[q];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t e = c0 + el + 4 * g + i;
          if (S[i] >= tr && e < a.N) {
            const uint32_t slot = atomicAdd(&lcnt[q], 1u);
            if (slot < (uint32_t)a.region)
              st_c<true>(a.cand + ((int64_t)q * a.chunks + blk) * a.region + slot,
                         composite(score_key(S[i] * a.scale), (int)e));
          }
        }
      }
    }
  }
  __syncthreads();
  if (threadIdx.x < a.B) st_c<true>(a.cnt + (int64_t)threadIdx.x * a.chunks + blk, lcnt[threadIdx.x]);
  dec_publish(&bar->c[blk * kDecFlagStride], tag + 3u);

  // D. the selections: query q in block q, once every block's candidates are out
  if (blk < a.B) {
    dec_wait(bar, bar->c, gridDim.x, tag + 3u);
    final_query<T, kDecThreads, CAP, true>(a, blk, u.fin.cs, u.fin.hs, u.fin.coff, part, sh_digit, sh_above,
                                           sh_n, sh_over, sh_thr);
  }
}

// ------------------------------------------------------------------ host

// Group size: about 4k groups per query (so the k-th largest group maximum
// sits near the top quarter of the groups), at most kMaxGroups groups.
int topk_group_size(int64_t N, int k) {
  int64_t target = N / (4 * (int64_t)k);
  int gs = 4;
  while (gs < 64 && (int64_t)gs * 2 <= target) gs *= 2;
  while (gs < 64 && (N + gs - 1) / gs > kMaxGroups) gs *= 2;
  return gs;
}

// Launch geometry of the score passes, shared by the workspace query and the
// launcher: entry chunks of tiles_per_wave 16-entry tiles per wave (times 4
// when the waves split the chunk), and the candidate region of each (query,
// chunk).
struct TopkGeom { int GS, G, qpb, nqb, wq, qblocks, tpw, chunks, region, csize; };

static TopkGeom topk_geom(int64_t B, int64_t N, int k, bool per_seq) {
  TopkGeom g;
  g.GS = topk_group_size(N, k);
  g.G = (int)((N + g.GS - 1) / g.GS);
  g.nqb = per_seq ? 1 : (B <= 16 ? 1 : (B <= 32 ? 2 : 4));
  // many queries: the four waves of a block take a query set each and share
  // the entry tiles; otherwise they share the queries and split the entries
  g.wq = (!per_seq && B >= 1024) ? 4 : 1;
  g.qpb = per_seq ? 1 : 16 * g.nqb * g.wq;
  g.qblocks = (int)((B + g.qpb - 1) / g.qpb);
  const int min_tpw = g.GS >= 16 ? g.GS / 16 : 1;
  const int wsplit = g.wq == 4 ? 1 : 4;                      // waves splitting a chunk
  g.tpw = g.wq == 4 ? 256 : 64;
  while (g.tpw > min_tpw &&
         (int64_t)g.qblocks * ((N + (int64_t)g.tpw * 16 * wsplit - 1) / ((int64_t)g.tpw * 16 * wsplit)) < 1024)
    g.tpw /= 2;
  g.chunks = (int)((N + (int64_t)g.tpw * 16 * wsplit - 1) / ((int64_t)g.tpw * 16 * wsplit));
  // about 1.2k candidates per query are expected; give each chunk room for
  // 16x its share (at least 32 slots), capped by the chunk size
  int64_t r = (16 * (int64_t)k + g.chunks - 1) / g.chunks;
  r = r < 32 ? 32 : r;
  const int64_t csize = (int64_t)g.tpw * 16 * wsplit;
  g.region = (int)(r > csize ? csize : r);
  g.csize = (int)csize;
  return g;
}

size_t topk_workspace_bytes(int64_t B, int64_t N, int k) {
  // per-sequence keys use one query per block, which has the most chunks
  const TopkGeom g1 = topk_geom(B, N, k, false), g2 = topk_geom(B, N, k, true);
  const int64_t slots = (int64_t)g1.chunks * g1.region > (int64_t)g2.chunks * g2.region
                            ? (int64_t)g1.chunks * g1.region : (int64_t)g2.chunks * g2.region;
  const int64_t chunks = g1.chunks > g2.chunks ? g1.chunks : g2.chunks;
  size_t bytes = 0;
  bytes += (size_t)B * slots * 8;                       // candidate regions
  bytes += (size_t)B * g1.G * 4;                        // group maxima
  bytes += (size_t)B * 4;                               // thresholds
  bytes += (size_t)B * chunks * 4;                      // counts per (query, chunk)
  return bytes + 256;
}

size_t topk_stored_score_bytes(int64_t B, int64_t N) {
  return (size_t)B * ((N + 15) / 16 * 16) * 4 + 256;
}

// below this many queries the per-query kernels take 1024 threads a block
constexpr int64_t kWideBelow = 256;

int topk_max_k() { return kMaxK; }
int64_t topk_max_entries() { return (int64_t)kMaxGroups * 64; }

// Per-device record of the stream that one-launch selections run on (see
// below).
constexpr int kDecDevices = 64;
struct DecodeGuard {
  std::mutex mu;
  bool used = false, several = false;
  hipStream_t stream = nullptr;
  uint64_t seq = 0;                                          // launches so far
};
static DecodeGuard& decode_guard(int dev) {
  static DecodeGuard guards[kDecDevices];
  return guards[dev];
}

// The tag of a device's n-th launch: a 64-bit mix (splitmix64's finaliser)
// of a per-process random salt, the device and n.  Successive tags differ by
// far more than the 3 their phases add.
static uint64_t decode_salt() {
  uint64_t s = 0;
  try {
    std::random_device rd;
    s = ((uint64_t)rd() << 32) ^ (uint64_t)rd();
  } catch (...) {
  }
  // also the clock and an address, should the random device give nothing
  s ^= (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count();
  s ^= (uint64_t)(uintptr_t)&s << 17;
  return s;
}
static uint64_t decode_tag(int dev, uint64_t n) {
  static const uint64_t salt = decode_salt();
  uint64_t z = salt + 0x9e3779b97f4a7c15ull * (n + ((uint64_t)dev << 48));
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}

// The fused decode selection when it applies: shared, fully visible keys;
// up to 32 queries; one resident block a compute unit holding its keys' raw
// scores in LDS; its workspace layout within topk_workspace_bytes.  Returns
// hipErrorNotSupported (nothing launched) when it does not apply.
template <class T>
static hipError_t launch_decode_fused(const TopkParams& p, IdxArgs a, void* ws, hipStream_t stream) {
  if (p.B > 32 || p.k > kMaxK) return hipErrorNotSupported;
  const int nqb = p.B <= 16 ? 1 : 2;
  // Not under stream capture: the multi-launch path is captured instead
  // (a replayed graph runs whenever its caller launches it, with no record
  // below to keep two of these kernels apart).
  int dev = 0, cus = 0;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0 ||
      hipStreamIsCapturing(stream, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone ||
      dev < 0 || dev >= kDecDevices)
    return hipErrorNotSupported;
  // keys a block: a multiple of 256 (whole 16-key tiles for its 16 waves)
  // and of 16 GS (each wave's keys hold whole groups), as few blocks as give
  // every compute unit at most one
  const int64_t unit = 16 * (int64_t)a.GS > 256 ? 16 * (int64_t)a.GS : 256;
  const int64_t C = ((p.N + cus - 1) / cus + unit - 1) / unit * unit;
  const int64_t nb = (p.N + C - 1) / C;
  // at least one block a query (a block takes one query's threshold and
  // selection)
  if (16 * nqb * (C + kDecPad) > kDecScores || nb < p.B || nb < 2 || nb > kDecMaxBlocks)
    return hipErrorNotSupported;
  const void* kern = nullptr;
  const bool small = p.k <= 1024;
  if (nqb == 1) kern = small ? (const void*)idx_decode_kernel<T, 1, 2048> : (const void*)idx_decode_kernel<T, 1, kCap>;
  else kern = small ? (const void*)idx_decode_kernel<T, 2, 2048> : (const void*)idx_decode_kernel<T, 2, kCap>;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kDecThreads, 0) != hipSuccess ||
      (int64_t)per_cu * cus < nb)
    return hipErrorNotSupported;
  // candidate regions: room for 16x each block's share of about 1.2k, at
  // least 32 slots, at most the block's keys
  int64_t r = (16 * (int64_t)p.k + nb - 1) / nb;
  r = r < 32 ? 32 : (r > C ? C : r);
  a.chunks = (int)nb;
  a.region = (int)r;
  a.csize = (int)C;
  a.cmagic = 0xffffffffu / (uint32_t)C;
  char* w = (char*)ws;
  a.cand = (uint64_t*)w;            w += (size_t)p.B * nb * r * 8;
  a.gmax = (uint32_t*)w;            w += (size_t)p.B * a.G * 4;
  a.thr = (uint32_t*)w;             w += (size_t)p.B * 4;
  a.cnt = (uint32_t*)w;             w += (size_t)p.B * nb * 4;
  w = (char*)(((uintptr_t)w + 255) & ~(uintptr_t)255);
  DecodeBar* bar = (DecodeBar*)w;   w += sizeof(DecodeBar);
  if ((size_t)(w - (char*)ws) > topk_workspace_bytes(p.B, p.N, p.k)) return hipErrorNotSupported;
  a.sraw = nullptr;
  // Two of these kernels must not run at once: each could hold part of
  // the chip while it waits for blocks of its own that cannot start.  They
  // therefore run on one stream per device, whose order keeps them apart:
  // the first call's.  Once a call comes on another stream, this and every
  // later selection on the device take the multi-launch path.  (Kernels of
  // other kinds running beside one only delay its waits: their blocks
  // finish and free their compute units.)
  DecodeGuard& gd = decode_guard(dev);
  uint64_t tag;
  try {                                                      // nothing may throw past the C entry points
    std::lock_guard<std::mutex> lock(gd.mu);
    if (!gd.used) {
      gd.used = true;
      gd.stream = stream;
    } else if (gd.stream != stream) {
      gd.several = true;
    }
    if (gd.several) return hipErrorNotSupported;
    tag = decode_tag(dev, ++gd.seq);
  } catch (...) {
    return hipErrorNotSupported;
  }
#define CSKV_DECODE(NQB, CAPV) \
  hipLaunchKernelGGL((idx_decode_kernel<T, NQB, CAPV>), dim3((unsigned)nb), dim3(kDecThreads), 0, stream, a, (int)C, bar, tag)
  if (nqb == 1 && small) CSKV_DECODE(1, 2048);
  else if (nqb == 1) CSKV_DECODE(1, kCap);
  else if (small) CSKV_DECODE(2, 2048);
  else CSKV_DECODE(2, kCap);
#undef CSKV_DECODE
  return hipGetLastError();
}

template <class T>
static hipError_t launch_topk_t(const TopkParams& p, void* ws, hipStream_t stream) {
  IdxArgs a;
  a.q = p.q; a.keys = p.keys; a.q_pos = p.q_pos; a.key_bstride = p.key_bstride;
  a.qsc = p.qsc; a.ksc = p.ksc;
  a.B = (int)p.B; a.N = (int)p.N; a.k = p.k; a.m = p.m; a.scale = p.scale; a.out = p.out;
  const bool per_seq = p.key_bstride != 0;
  const TopkGeom g = topk_geom(p.B, p.N, p.k, per_seq);
  a.GS = g.GS; a.G = g.G; a.qpb = g.qpb; a.tiles_per_wave = g.tpw;
  a.gs_shift = 0;
  while ((1 << a.gs_shift) < g.GS) ++a.gs_shift;             // group sizes are powers of two
  a.chunks = g.chunks; a.region = g.region;
  a.csize = g.csize; a.cmagic = 0xffffffffu / (uint32_t)g.csize;
  char* w = (char*)ws;
  a.cand = (uint64_t*)w;            w += (size_t)p.B * g.chunks * g.region * 8;
  a.gmax = (uint32_t*)w;            w += (size_t)p.B * a.G * 4;
  a.thr = (uint32_t*)w;             w += (size_t)p.B * 4;
  a.cnt = (uint32_t*)w;
  // per-sequence keys with room in the workspace: keep the raw scores
  const size_t base = topk_workspace_bytes(p.B, p.N, p.k);
  a.sraw = nullptr;
  a.np = (p.N + 15) / 16 * 16;
  if (per_seq && p.ws_bytes >= base + topk_stored_score_bytes(p.B, p.N))
    a.sraw = (float*)((char*)ws + (base + 255) / 256 * 256);
  const int nqb = g.nqb, qblocks = g.qblocks, chunks = g.chunks;
  dim3 grid(chunks, qblocks);
#define CSKV_SCORE(NQB, MODE, WQ) \
  hipLaunchKernelGGL((idx_score_kernel<T, NQB, MODE, WQ>), grid, dim3(256), 0, stream, a)
  // many queries on 32x32 tiles (fp8, bf16, MXFP4 keys; groups of >= 32)
  constexpr bool kTile32 = !std::is_same<T, float>::value;
  const bool tile32 = kTile32 && g.wq == 4 && g.GS >= 32;
#define CSKV_SCORE32(MODE)                                                                     \
  {                                                                                            \
    if (MODE == 1 || g.GS == 64)                                                               \
      hipLaunchKernelGGL((idx_score32_kernel<T, 2, MODE, 6>), grid, dim3(256), 0, stream, a);  \
    else                                                                                       \
      hipLaunchKernelGGL((idx_score32_kernel<T, 2, MODE, 5>), grid, dim3(256), 0, stream, a);  \
  }
#define CSKV_SCORE_PASS(MODE)                                                  \
  if (tile32) { if constexpr (kTile32) { CSKV_SCORE32(MODE) } }               \
  else if (g.wq == 4) CSKV_SCORE(4, MODE, 4);                                  \
  else if (nqb == 1) CSKV_SCORE(1, MODE, 1);                                   \
  else if (nqb == 2) CSKV_SCORE(2, MODE, 1);                                   \
  else CSKV_SCORE(4, MODE, 1)
  // one block per query for the threshold and the final selection: 1024
  // threads when there are fewer queries than compute units (decode), so
  // that each query's serial steps run on a whole compute unit; 256 threads
  // otherwise (two blocks per compute unit)
  const bool wide = p.B < kWideBelow;
  if (!per_seq && !p.q_pos) {
    const hipError_t e = launch_decode_fused<T>(p, a, ws, stream);
    if (e != hipErrorNotSupported) return e;
  }
  CSKV_SCORE_PASS(0);
  if (wide) hipLaunchKernelGGL(idx_threshold_kernel<1024>, dim3((unsigned)p.B), dim3(1024), 0, stream, a);
  else hipLaunchKernelGGL(idx_threshold_kernel<256>, dim3((unsigned)p.B), dim3(256), 0, stream, a);
  if (a.sraw)
    hipLaunchKernelGGL(idx_collect_kept_kernel, grid, dim3(256), 0, stream, a);
  else
    CSKV_SCORE_PASS(1);
#undef CSKV_SCORE_PASS
#undef CSKV_SCORE32
#undef CSKV_SCORE
  const bool small = p.k <= 1024;                            // 2048 candidates in LDS
  if (wide && small)
    hipLaunchKernelGGL((idx_final_kernel<T, 1024, 2048>), dim3((unsigned)p.B), dim3(1024), 0, stream, a);
  else if (wide)
    hipLaunchKernelGGL((idx_final_kernel<T, 1024, kCap>), dim3((unsigned)p.B), dim3(1024), 0, stream, a);
  else if (small)
    hipLaunchKernelGGL((idx_final_kernel<T, 256, 2048>), dim3((unsigned)p.B), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((idx_final_kernel<T, 256, kCap>), dim3((unsigned)p.B), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_topk(const TopkParams& p, void* ws, hipStream_t stream) {
  if (p.dt == 0) return launch_topk_t<float>(p, ws, stream);
  if (p.dt == 1) return launch_topk_t<bf16_t>(p, ws, stream);
  if (p.dt == 3) return launch_topk_t<fp4x2_t>(p, ws, stream);
  return launch_topk_t<e4m3_t>(p, ws, stream);
}

}  // namespace cskv
