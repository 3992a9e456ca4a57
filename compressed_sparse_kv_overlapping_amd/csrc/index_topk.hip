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
template <> struct Frag<fp4x2_t> { uint32_t v; uint32_t s; };  // 8 codes; block scale as fp32 bits

// Bytes of a 64-element row, and the fragment type the MFMA consumes.
// MXFP4 is decoded to bf16, which is exact: an E2M1 value times a power of
// two has at most two significant bits (within bf16's exponent range).
template <class T> struct Elem {
  static constexpr int kRowBytes = 64 * (int)sizeof(T);
  using QF = Frag<T>;
};
template <> struct Elem<fp4x2_t> {
  static constexpr int kRowBytes = 32;
  using QF = Frag<bf16_t>;
};

// 8 E2M1 codes times their block scale, as 8 bf16 (gfx950 converts two
// codes per instruction).  Queries and keys go through the same conversion,
// so the pairing of slots in a dot product never depends on which nibble a
// converted pair puts first.
__device__ __forceinline__ void fp4_decode(Frag<bf16_t>& d, const Frag<fp4x2_t>& f) {
  d.v = fp4x8_to_bf16(f.v, __uint_as_float(f.s));
}

// Key fragments as the MFMA takes them (a copy, or the MXFP4 decode).
template <class T>
__device__ __forceinline__ void key_decode(typename Elem<T>::QF* d, const Frag<T>* k) {
  d[0] = k[0];
  d[1] = k[1];
}
template <>
__device__ __forceinline__ void key_decode<fp4x2_t>(Frag<bf16_t>* d, const Frag<fp4x2_t>* k) {
  fp4_decode(d[0], k[0]);
  fp4_decode(d[1], k[1]);
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
  const char* p = kb + r * 32;
  f[0].v = *reinterpret_cast<const uint32_t*>(p + 4 * g);
  f[1].v = *reinterpret_cast<const uint32_t*>(p + 16 + 4 * g);
  const uint32_t s2 = *reinterpret_cast<const uint16_t*>(sb + 2 * r);
  f[0].s = e8m0_f32_bits(s2 & 255u);
  f[1].s = e8m0_f32_bits(s2 >> 8);
}

// The block scales of row r for fragments whose codes came from LDS.
template <class T>
__device__ __forceinline__ void key_scales(Frag<T>* f, const uint8_t* sb, int64_t r) {}
template <>
__device__ __forceinline__ void key_scales<fp4x2_t>(Frag<fp4x2_t>* f, const uint8_t* sb, int64_t r) {
  const uint32_t s2 = *reinterpret_cast<const uint16_t*>(sb + 2 * r);
  f[0].s = e8m0_f32_bits(s2 & 255u);
  f[1].s = e8m0_f32_bits(s2 >> 8);
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
  static __device__ __forceinline__ int frag_off(int ks, int g) { return (32 * ks + 8 * g) * kRow / 64; }
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
      mma16(S[j], kd[0], qf[j][0]);
      mma16(S[j], kd[1], qf[j][1]);
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
        key_scales<T>(f, sbase, row < a.N ? row : a.N - 1);
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

// A lower bound of the k-th largest of the G group maxima of each query (0
// if fewer than k non-empty groups or fewer than k visible entries).  The
// maxima are read from L2; only the histogram lives in LDS.
template <int NT>
__global__ __launch_bounds__(NT) void idx_threshold_kernel(IdxArgs a) {
  __shared__ uint32_t hist[4096], part[NT / 32];
  __shared__ uint32_t sh_digit, sh_above;
  const int b = blockIdx.x;
  const uint32_t* gm = a.gmax + (int64_t)b * a.G;
  uint32_t ne = 0, mn = 0xffffffffu, mx = 0u;
  for (int i = threadIdx.x; i < a.G; i += NT) {
    const uint32_t v = gm[i];
    if (v != 0u) { ++ne; mn = min(mn, v); mx = max(mx, v); }
  }
  uint32_t nonempty;
  block_excl_scan<NT>(ne, part, &nonempty);
  uint32_t lo, hi;
  block_minmax<NT>(mn, mx, part, &lo, &hi);
  const int nv = n_visible(a, b);
  if (nv <= a.k || nonempty < (uint32_t)a.k) {
    if (threadIdx.x == 0) a.thr[b] = 0u;
    return;
  }
  // one pass over 4096 bins of the key range: the lower edge of the bin that
  // holds the k-th largest maximum is at most that maximum, so at least k
  // groups (hence k entries) still reach it; a bin's width of extra
  // candidates is all it costs
  const uint32_t range = hi - lo;
  const int bits = range ? 32 - __clz((int)range) : 0;     // range < 2^bits
  const int shift = bits > 12 ? bits - 12 : 0;
  for (int i = threadIdx.x; i < 4096; i += NT) hist[i] = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < a.G; i += NT) {
    const uint32_t v = gm[i];
    if (v != 0u) atomicAdd(&hist[(v - lo) >> shift], 1u);
  }
  __syncthreads();
  find_kth_bin<NT>(hist, 4096, (uint32_t)a.k, &sh_digit, &sh_above, part);
  if (threadIdx.x == 0) a.thr[b] = lo + (sh_digit << shift);
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
// crowded bin falls back to further passes).  Each selected candidate is then
// written at its chunk's output offset plus its rank by index among the
// chunk's selected ones, so the output is ascending without a global sort.
constexpr int kMaxChunks = 2048;
constexpr int kFinalBB = 11;                 // histogram of 2^11 bins
constexpr int kMem = 512;                    // bin members ranked exactly
template <class T, int NT>
__global__ __launch_bounds__(NT) void idx_final_kernel(IdxArgs a) {
  // candidates (list) or, on overflow, the k selected indices
  __shared__ union { uint64_t cand[kCap]; int32_t sel[kMaxK]; } cs;
  // the histogram, then the members of the k-th bin, then the chunks' output
  // offsets
  __shared__ union { uint32_t hist[1 << kFinalBB]; uint64_t mem[kMem]; uint16_t csel[kMaxChunks]; } hs;
  __shared__ uint16_t coff[kMaxChunks + 1];                  // list offset of each chunk
  __shared__ uint32_t part[NT / 32];
  __shared__ uint32_t sh_digit, sh_above, sh_nsel, sh_over;
  __shared__ uint64_t sh_thr;
  uint64_t* cand = cs.cand;
  int32_t* sel = cs.sel;
  uint32_t* hist = hs.hist;
  const int b = blockIdx.x;
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
    const uint32_t n = a.cnt[(int64_t)b * a.chunks + c];
    full |= n > (uint32_t)a.region;
    mine += n > (uint32_t)a.region ? (uint32_t)a.region : n;
  }
  __syncthreads();
  if (full) sh_over = 1;
  uint32_t total;
  const uint32_t base = block_excl_scan<NT>(mine, part, &total);
  const bool overflow = sh_over != 0 || total > (uint32_t)kCap;
  if (!overflow) {
    // chunk offsets in the list, then a copy spread over the whole block:
    // list slot j belongs to the last chunk whose offset is <= j
    uint32_t at = base;
    for (int c = c0; c < c1; ++c) {
      coff[c] = (uint16_t)at;
      const uint32_t n = a.cnt[(int64_t)b * a.chunks + c];
      at += n > (uint32_t)a.region ? (uint32_t)a.region : n;
    }
    if (t == 0) coff[a.chunks] = (uint16_t)total;
    __syncthreads();
    for (uint32_t j = t; j < total; j += NT) {
      int lo = 0, hi = a.chunks;                             // coff[lo] <= j < coff[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (coff[mid] <= j) lo = mid; else hi = mid;
      }
      cand[j] = a.cand[((int64_t)b * a.chunks + lo) * a.region + (j - coff[lo])];
    }
  }
  const int nc = overflow ? 0 : (int)total;
  __syncthreads();

  // the k-th largest composite
  uint64_t prefix = 0;
  if (!overflow) {
    uint32_t mn = 0xffffffffu, mx = 0u;
    for (int j = t; j < nc; j += NT) {
      const uint32_t h = (uint32_t)(cand[j] >> 32);
      mn = min(mn, h);
      mx = max(mx, h);
    }
    uint32_t lo, hi;
    block_minmax<NT>(mn, mx, part, &lo, &hi);
    const uint32_t range = hi - lo;
    const int bits = range ? 32 - __clz((int)range) : 0;   // range < 2^bits
    const int shift = bits > kFinalBB ? bits - kFinalBB : 0;
    for (int i = t; i < (1 << kFinalBB); i += NT) hist[i] = 0;
    if (t == 0) { sh_nsel = 0; sh_thr = 0; }
    __syncthreads();
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
      __syncthreads();                                       // hist is read; csel reuses it
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
    // per-chunk counts of selected candidates -> output offsets; then each
    // selected candidate goes to its chunk's offset plus its rank by index
    // among the chunk's selected ones (chunks are ascending entry ranges)
    uint32_t mine_sel = 0;
    for (int c = c0; c < c1; ++c) {
      uint32_t m = 0;
      for (uint32_t j = coff[c]; j < coff[c + 1]; ++j) m += cand[j] >= thr;
      hs.csel[c] = (uint16_t)m;
      mine_sel += m;
    }
    uint32_t nsel;
    uint32_t ob = block_excl_scan<NT>(mine_sel, part, &nsel);
    for (int c = c0; c < c1; ++c) {
      const uint32_t m = hs.csel[c];
      hs.csel[c] = (uint16_t)ob;
      ob += m;
    }
    __syncthreads();
    for (uint32_t j = t; j < total; j += NT) {
      const uint64_t v = cand[j];
      if (v < thr) continue;
      int lo = 0, hi = a.chunks;                             // chunk of slot j
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (coff[mid] <= j) lo = mid; else hi = mid;
      }
      uint32_t rank = 0;                                     // selected with a smaller index
      for (uint32_t i = coff[lo]; i < coff[lo + 1]; ++i) {
        const uint64_t w = cand[i];
        rank += (w >= thr) && ((uint32_t)w > (uint32_t)v);  // larger low word = smaller index
      }
      const uint32_t o = hs.csel[lo] + rank;
      if (o < (uint32_t)a.k) out[o] = (int32_t)(0xffffffffu - (uint32_t)v);
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
      if (at < (uint32_t)kMaxK) sel[at] = e;
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
struct TopkGeom { int GS, G, qpb, nqb, wq, qblocks, tpw, chunks, region; };

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
#define CSKV_SCORE_PASS(MODE)                                                  \
  if (g.wq == 4) CSKV_SCORE(4, MODE, 4);                                       \
  else if (nqb == 1) CSKV_SCORE(1, MODE, 1);                                   \
  else if (nqb == 2) CSKV_SCORE(2, MODE, 1);                                   \
  else CSKV_SCORE(4, MODE, 1)
  // one block per query for the threshold and the final selection: 1024
  // threads when there are fewer queries than compute units (decode), so
  // that each query's serial steps run on a whole compute unit; 256 threads
  // otherwise (two blocks per compute unit)
  const bool wide = p.B < kWideBelow;
  CSKV_SCORE_PASS(0);
  if (wide) hipLaunchKernelGGL(idx_threshold_kernel<1024>, dim3((unsigned)p.B), dim3(1024), 0, stream, a);
  else hipLaunchKernelGGL(idx_threshold_kernel<256>, dim3((unsigned)p.B), dim3(256), 0, stream, a);
  if (a.sraw)
    hipLaunchKernelGGL(idx_collect_kept_kernel, grid, dim3(256), 0, stream, a);
  else
    CSKV_SCORE_PASS(1);
#undef CSKV_SCORE_PASS
#undef CSKV_SCORE
  if (wide) hipLaunchKernelGGL((idx_final_kernel<T, 1024>), dim3((unsigned)p.B), dim3(1024), 0, stream, a);
  else hipLaunchKernelGGL((idx_final_kernel<T, 256>), dim3((unsigned)p.B), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_topk(const TopkParams& p, void* ws, hipStream_t stream) {
  if (p.dt == 0) return launch_topk_t<float>(p, ws, stream);
  if (p.dt == 1) return launch_topk_t<bf16_t>(p, ws, stream);
  if (p.dt == 3) return launch_topk_t<fp4x2_t>(p, ws, stream);
  return launch_topk_t<e4m3_t>(p, ws, stream);
}

}  // namespace cskv
