// Split-KV decode attention over gathered rows (CSA) or all entries (HCA),
// and the cross-split merge, for gfx950.
//
// Method: "Frontier Techniques: NTK RoPE, CSA+HCA, QAT, MTP" 2.1 (attention
// over the top entries plus a 128-token raw window) and 2.2 (dense attention
// over all heavily compressed entries); "DeepSeek V4 comprimeix el context",
// sections "CSA: buscar primer i atendre despres" and "HCA: un resum global
// 128 vegades mes curt".  Rows are 576 wide: logits use all 576 dims, the
// value is dims 0..511 (shared-KV layout of 512 latent dims plus a 64-dim
// RoPE part, "The State and Signal Problem", section "MLA compresses what
// generation must remember").  All heads read the same rows.
//
// Kernel shape: a block handles one query, a group of heads and one split of
// that query's rows.  Rows arrive in tiles of 32: the block gathers them into
// LDS twice, row-major (K, for the logits) and transposed (V^T, for the
// weighted sum).  Each wave owns HB blocks of 16 heads (16x16x32 bf16 MFMA,
// or 16x16x4 fp32) and keeps their queries and output accumulators in
// registers.  Per tile:
//   S^T[rows, heads] = K_tile . Q^T            (MFMA, A = K from LDS)
//   online softmax per head (exp2 domain)
//   O^T[d, heads]   += V^T_tile . P^T           (MFMA, A = V^T from LDS)
// The accumulator layout of S^T is used directly as the B operand of the
// second product: its k-slots are assigned to rows in the order the first
// product leaves them in each lane.  With one split the block writes the
// final output; otherwise it writes a normalised partial and its lse, and
// the merge kernel combines the splits.
#include "common.hpp"
#include "kernels.hpp"

namespace cskv {

constexpr int kE = 576, kDv = 512, kTile = 32;
constexpr float kLazy = 8.f;
constexpr float kRefBand = 64.f;

template <class T> struct AttnCfg;
template <> struct AttnCfg<bf16_t> {
  static constexpr int NW = 4;                               // 64 or 128 heads per block
  static constexpr int EPC = 8;                              // elements per 16-byte chunk
  static constexpr int KP = kE + 8;                          // K tile row pitch (elements)
  static constexpr int VP = kTile + 4;                       // V^T row pitch (elements)
};
template <> struct AttnCfg<float> {
  static constexpr int NW = 1;                               // 16 heads per block
  static constexpr int EPC = 8;
  static constexpr int KP = kE + 4;
  static constexpr int VP = kTile + 4;
};

struct AttnArgs {
  const void* q;
  const void* entries;
  const void* window;
  const int32_t* idx;        // selected entries (CSA)
  const int64_t* q_pos;      // NULL: decode window
  int64_t ent_bstride, win_bstride, win_pos0, win_rows, N;
  int dense;                 // 1: all N entries, no window (HCA)
  int B, H, W, k, nslots, slots_per_split, nsplit;
  float c;                   // scale * log2(e)
  void* out;                 // [B][H][512] when nsplit == 1
  float* lse;                // [B][H] (nullable)
  float* o_part;             // [B][H][nsplit][512]
  float* lse_part;           // [B][H][nsplit]
};

// Keeps the scheduler from hoisting every LDS fragment load of an unrolled
// loop to its top (which would need more registers than a wave has).
__device__ __forceinline__ void fence_sched() { asm volatile("" ::: "memory"); }

// Element-typed 8-wide register chunk, used for the transposed V writes.
template <class T> struct Chunk8;
template <> struct Chunk8<bf16_t> {
  uint4 v;
  __device__ __forceinline__ void load(const bf16_t* p) { v = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void zero() { v = make_uint4(0, 0, 0, 0); }
  __device__ __forceinline__ void store(bf16_t* p) const { *reinterpret_cast<uint4*>(p) = v; }
  __device__ __forceinline__ uint16_t get(int t) const {
    uint32_t w = t < 2 ? v.x : t < 4 ? v.y : t < 6 ? v.z : v.w;
    return (t & 1) ? (uint16_t)(w >> 16) : (uint16_t)(w & 0xffff);
  }
};
template <> struct Chunk8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = reinterpret_cast<const float4*>(p)[0];
    b = reinterpret_cast<const float4*>(p)[1];
  }
  __device__ __forceinline__ void zero() { a = b = make_float4(0.f, 0.f, 0.f, 0.f); }
  __device__ __forceinline__ void store(float* p) const {
    reinterpret_cast<float4*>(p)[0] = a;
    reinterpret_cast<float4*>(p)[1] = b;
  }
  __device__ __forceinline__ float get(int t) const {
    return t == 0 ? a.x : t == 1 ? a.y : t == 2 ? a.z : t == 3 ? a.w
         : t == 4 ? b.x : t == 5 ? b.y : t == 6 ? b.z : b.w;
  }
};

// 4 consecutive rows of one V^T line (8 bytes bf16, 16 bytes fp32).
template <class T> struct Quad;
template <> struct Quad<bf16_t> {
  static __device__ __forceinline__ void store(bf16_t* p, const Chunk8<bf16_t> c[4], int t) {
    uint32_t lo = (uint32_t)c[0].get(t) | ((uint32_t)c[1].get(t) << 16);
    uint32_t hi = (uint32_t)c[2].get(t) | ((uint32_t)c[3].get(t) << 16);
    *reinterpret_cast<uint2*>(p) = make_uint2(lo, hi);
  }
};
template <> struct Quad<float> {
  static __device__ __forceinline__ void store(float* p, const Chunk8<float> c[4], int t) {
    *reinterpret_cast<float4*>(p) = make_float4(c[0].get(t), c[1].get(t), c[2].get(t), c[3].get(t));
  }
};

// Fragment of V^T for the second product: rows r0..r0+3 and r1..r1+3 of
// line d (two 4-row quads).
__device__ __forceinline__ void vt_frag(Frag<bf16_t>& f, const bf16_t* line, int r0, int r1) {
  uint2 a = *reinterpret_cast<const uint2*>(line + r0);
  uint2 b = *reinterpret_cast<const uint2*>(line + r1);
  f.v = u32x4{a.x, a.y, b.x, b.y};
}
__device__ __forceinline__ void vt_frag(Frag<float>& f, const float* line, int r0, int r1) {
  float4 a = *reinterpret_cast<const float4*>(line + r0);
  float4 b = *reinterpret_cast<const float4*>(line + r1);
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
  f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}

__device__ __forceinline__ void p_frag(Frag<bf16_t>& f, const float* p) {
  f.v = u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
              pack_bf16x2(p[6], p[7])};
}
__device__ __forceinline__ void p_frag(Frag<float>& f, const float* p) {
#pragma unroll
  for (int t = 0; t < 8; ++t) f.v[t] = p[t];
}

template <class T>
__device__ __forceinline__ void store_out4(T* p, float a, float b, float c, float d);
template <> __device__ __forceinline__ void store_out4<bf16_t>(bf16_t* p, float a, float b, float c,
                                                               float d) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
}
template <> __device__ __forceinline__ void store_out4<float>(float* p, float a, float b, float c,
                                                              float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}

// Row (within a 32-row tile) held by logit value i (0..7) of lane group g:
// two 16-row MFMA tiles stacked, values 0..3 in the first, 4..7 in the second.
__device__ __forceinline__ int srow(int g, int i) { return 16 * (i >> 2) + 4 * g + (i & 3); }

// HB = head blocks of 16 per wave.  With HB = 2 every K and V^T fragment read
// from LDS feeds two MFMAs, which halves the LDS traffic per flop.
template <class T, int HB>
__global__ __launch_bounds__(64 * AttnCfg<T>::NW) void attend_kernel(AttnArgs a) {
  typedef AttnCfg<T> C;
  constexpr int MN = 16, NW = C::NW, NT = 64 * NW;
  constexpr int KSTEP = 32;                                  // contraction per MFMA step
  constexpr int NKS = kE / KSTEP;
  constexpr int NDB = kDv / MN;                              // output d-blocks
  __shared__ __attribute__((aligned(16))) T Ks[kTile * C::KP];
  __shared__ __attribute__((aligned(16))) T Vt[kDv * C::VP];
  __shared__ int64_t row_off[2][kTile];
  __shared__ int row_ok[2][kTile];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int split = blockIdx.x, hg = blockIdx.y, b = blockIdx.z;
  const int col = lane % MN, g = lane / MN;
  int hh[HB];
  bool hok[HB];
#pragma unroll
  for (int j = 0; j < HB; ++j) {
    hh[j] = ((hg * NW + wave) * HB + j) * MN + col;
    hok[j] = hh[j] < a.H;
  }
  const T* q = reinterpret_cast<const T*>(a.q);
  const T* ent = reinterpret_cast<const T*>(a.entries);
  const T* win = reinterpret_cast<const T*>(a.window);

  // query fragments of this lane's heads: k-slots (g, t) <-> dim 32*ks + 8g + t
  Frag<T> qf[HB][NKS];
#pragma unroll
  for (int j = 0; j < HB; ++j) {
    const T* qp = q + ((int64_t)b * a.H + (hok[j] ? hh[j] : 0)) * kE;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      frag_load(qf[j][ks], qp + ks * KSTEP + 8 * g);
      if (!hok[j]) {
        Frag<T> z{};
        qf[j][ks] = z;
      }
    }
  }
  f32x4 O[HB][NDB];
#pragma unroll
  for (int j = 0; j < HB; ++j)
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) O[j][db][i] = 0.f;
  float m_run[HB], l_run[HB];
#pragma unroll
  for (int j = 0; j < HB; ++j) { m_run[j] = -INFINITY; l_run[j] = 0.f; }

  // window rows of this query: buffer row of its first row, and count
  int64_t win_row0 = 0;
  int nwin = a.W;
  if (a.q_pos) {
    const int64_t pos = a.q_pos[b];
    int64_t lo = pos - a.W + 1;
    if (lo < 0) lo = 0;
    nwin = (int)(pos - lo + 1);
    win_row0 = lo - a.win_pos0;
  }
  const int s_begin = split * a.slots_per_split;
  const int s_end = min(a.nslots, s_begin + a.slots_per_split);

  // Software pipeline: while tile i is multiplied out of LDS, the rows of
  // tile i+1 are already in flight into registers (their addresses were
  // resolved into the other row_off slot).
  constexpr int kVTasks = 8 * (kDv / 8);                      // 4-row x 8-dim value tasks
  constexpr int kRTasks = kTile * ((kE - kDv) / 8);           // RoPE chunks
  constexpr int kVPer = (kVTasks + NT - 1) / NT, kRPer = (kRTasks + NT - 1) / NT;
  auto resolve = [&](int t0, int slot) {
    if (threadIdx.x < kTile) {
      const int s = t0 + threadIdx.x;
      int64_t off = 0;
      int ok = 0;
      if (s < s_end) {
        if (a.dense) {
          ok = 1;
          off = (int64_t)b * a.ent_bstride + (int64_t)s * kE;
        } else if (s < a.k) {
          const int e = a.idx[(int64_t)b * a.k + s];
          ok = (e >= 0 && e < a.N);                            // -1 (or out of range): no row
          off = (int64_t)b * a.ent_bstride + (int64_t)(ok ? e : 0) * kE;
        } else {
          const int w = s - a.k;
          const int64_t r = win_row0 + w;
          ok = w < nwin && r >= 0 && r < a.win_rows;           // rows outside the buffer are skipped
          off = -1 - ((int64_t)b * a.win_bstride + (ok ? r : 0) * kE);   // negative: window row
        }
      }
      row_off[slot][threadIdx.x] = off;
      row_ok[slot][threadIdx.x] = ok;
    }
  };
  Chunk8<T> pv[kVPer][4], pr[kRPer];
  auto fetch = [&](int slot) {
#pragma unroll
    for (int u = 0; u < kVPer; ++u) {
      const int task = threadIdx.x + u * NT;
      const int qd = task & 7, cc = (task >> 3) & 63;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * qd + i;
        if (task < kVTasks && row_ok[slot][r]) {
          const int64_t off = row_off[slot][r];
          const T* src = off >= 0 ? ent + off : win + (-1 - off);
          pv[u][i].load(src + cc * 8);
        } else {
          pv[u][i].zero();
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kRPer; ++u) {
      const int task = threadIdx.x + u * NT;
      const int r = (task >> 3) & (kTile - 1), cc = kDv / 8 + (task & 7);
      if (task < kRTasks && row_ok[slot][r]) {
        const int64_t off = row_off[slot][r];
        const T* src = off >= 0 ? ent + off : win + (-1 - off);
        pr[u].load(src + cc * 8);
      } else {
        pr[u].zero();
      }
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int u = 0; u < kVPer; ++u) {
      const int task = threadIdx.x + u * NT;
      if (task < kVTasks) {
        const int qd = task & 7, cc = task >> 3;
#pragma unroll
        for (int i = 0; i < 4; ++i) pv[u][i].store(Ks + (4 * qd + i) * C::KP + cc * 8);
#pragma unroll
        for (int t = 0; t < 8; ++t) Quad<T>::store(Vt + (cc * 8 + t) * C::VP + 4 * qd, pv[u], t);
      }
    }
#pragma unroll
    for (int u = 0; u < kRPer; ++u) {
      const int task = threadIdx.x + u * NT;
      if (task < kRTasks) {
        const int r = task >> 3, cc = kDv / 8 + (task & 7);
        pr[u].store(Ks + r * C::KP + cc * 8);
      }
    }
  };
  // bf16 keeps the next tile in flight; fp32 (a single wave holding a whole
  // tile) fetches and stages back to back
  constexpr bool kOverlap = sizeof(T) == 2;
  int slot = 0;
  if (kOverlap && s_begin < s_end) {
    resolve(s_begin, 0);
    __syncthreads();
    fetch(0);
  }
  for (int t0 = s_begin; t0 < s_end; t0 += kTile) {
    if constexpr (kOverlap) {
      stage();                                                 // tile t0 -> LDS
      if (t0 + kTile < s_end) resolve(t0 + kTile, slot ^ 1);
      __syncthreads();
      if (t0 + kTile < s_end) fetch(slot ^ 1);                 // next tile in flight
    } else {
      resolve(t0, slot);
      __syncthreads();
      fetch(slot);
      stage();
      __syncthreads();
    }
    const int* tile_ok = row_ok[slot];
    // logits S^T[row, head]: rows 0..15 in S0, 16..31 in S1
    f32x4 S0[HB], S1[HB];
#pragma unroll
    for (int j = 0; j < HB; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) { S0[j][i] = 0.f; S1[j][i] = 0.f; }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      Frag<T> a0, a1;
      frag_load(a0, Ks + col * C::KP + ks * KSTEP + 8 * g);
      frag_load(a1, Ks + (16 + col) * C::KP + ks * KSTEP + 8 * g);
#pragma unroll
      for (int j = 0; j < HB; ++j) {
        mma16(S0[j], a0, qf[j][ks]);
        mma16(S1[j], a1, qf[j][ks]);
      }
      if (HB > 1 && (ks & 3) == 3) fence_sched();
    }
    // online softmax (per head = per lane column)
    Frag<T> pf[HB];
#pragma unroll
    for (int j = 0; j < HB; ++j) {
      float sv[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) { sv[i] = S0[j][i]; sv[4 + i] = S1[j][i]; }
      float tmax = -INFINITY;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        sv[i] = tile_ok[srow(g, i)] ? sv[i] * a.c : -INFINITY;
        tmax = fmaxf(tmax, sv[i]);
      }
      tmax = fmaxf(tmax, shfl_xor(tmax, 16));
      tmax = fmaxf(tmax, shfl_xor(tmax, 32));
      // Lazy rescaling: the reference max of a head only moves when the tile
      // max exceeds it by more than kLazy (log2 units), so weights stay below
      // 2^kLazy and the accumulators are rescaled rarely (wave-uniform branch).
      if (__any(tmax > m_run[j] + kLazy)) {
        const float m_new = fmaxf(m_run[j], tmax);
        const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run[j] - m_new);
        l_run[j] *= alpha;
        m_run[j] = m_new;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i) O[j][db][i] *= alpha;
      }
      const float m_use = (m_run[j] == -INFINITY) ? 0.f : m_run[j];
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        sv[i] = __builtin_amdgcn_exp2f(sv[i] - m_use);
        psum += sv[i];
      }
      l_run[j] += psum;
      p_frag(pf[j], sv);
    }

    // O^T[d, head] += V^T[d, rows] . P^T[rows, head]
    {
      const int r0 = 4 * g, r1 = 16 + 4 * g;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        Frag<T> vf;
        vt_frag(vf, Vt + (db * MN + col) * C::VP, r0, r1);
#pragma unroll
        for (int j = 0; j < HB; ++j) mma16(O[j][db], vf, pf[j]);
        if (HB > 1 && (db & 7) == 7) fence_sched();
      }
    }
    __syncthreads();
    if constexpr (kOverlap) slot ^= 1;
  }

  const float LN2 = 0.6931471805599453f;
#pragma unroll
  for (int j = 0; j < HB; ++j) {
    // total row sum of this head over the lane groups
    float l = l_run[j];
    l += shfl_xor(l, 16);
    l += shfl_xor(l, 32);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const float lse2 = l > 0.f ? m_run[j] + __log2f(l) : -INFINITY;
    if (!hok[j]) continue;
    const int h = hh[j];
    if (a.nsplit == 1) {
      T* o = reinterpret_cast<T*>(a.out) + ((int64_t)b * a.H + h) * kDv;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int d = db * MN + 4 * g;
        store_out4<T>(o + d, O[j][db][0] * inv, O[j][db][1] * inv, O[j][db][2] * inv,
                      O[j][db][3] * inv);
      }
      if (a.lse && g == 0) a.lse[(int64_t)b * a.H + h] = lse2 * LN2;
    } else {
      float* o = a.o_part + (((int64_t)b * a.H + h) * a.nsplit + split) * kDv;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int d = db * MN + 4 * g;
        store_out4<float>(o + d, O[j][db][0] * inv, O[j][db][1] * inv, O[j][db][2] * inv,
                          O[j][db][3] * inv);
      }
      if (g == 0) a.lse_part[((int64_t)b * a.H + h) * a.nsplit + split] = lse2 * LN2;
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 attention, 128 heads per block.
//
// A block of 4 waves takes 128 heads of one query and one split of its rows;
// each wave owns 32 heads (two 16-head MFMA blocks), so every K or V
// fragment read from LDS feeds two MFMAs.  A wave keeps its output
// accumulators (256 registers) and the queries of its first head block (72)
// in registers for the whole split; the queries of its second head block are
// read from LDS.  One wave per SIMD.
//
// Tiles are gathered from HBM straight into LDS (global_load_lds, 16 bytes
// per lane, no registers), one tile ahead into the other of two buffers.  A
// tile holds 32 rows x 72 chunks of 16 bytes.  Copy n fills slots
// [64 n, 64 n + 64): lanes 0..31 take chunk 2n of rows 0..31, lanes 32..63
// chunk 2n + 1 of the rows rotated by 8, so that chunk c of row r sits in slot
//   64 (c / 2) + 32 (c % 2) + ((r + 8 (c % 2)) % 32)
// and every lane copies a single row.  Both LDS read patterns then touch
// distinct banks (64 banks of 4 bytes, 16 lanes a pass):
//   logits: 16 rows x one chunk (ds_read_b128): one 256-byte run, or two
//           128-byte runs that do not alias,
//   values: 4 rows x two chunks, read transposed (ds_read_b64_tr_b16): runs in
//           distinct banks; the transposed read hands each lane four
//           consecutive rows of one value dimension, the A operand of
//           O^T += V^T P^T.
// The gather is issued from inline assembly, so the compiler does not see
// an LDS write in flight; the loop waits for it explicitly before the
// barrier that opens each tile.
//
// Softmax reference: a head's first visible tile sets it (its accumulators
// are still zero then) and it never moves, so the accumulators are never
// rescaled in the loop; later weights may reach 2^kRefBand, far inside fp32
// and bf16 range.  A logit beyond that band is flagged, and the block then
// runs the split again: first for each head's exact maximum, then
// accumulating against it.
constexpr int kWideWaves = 4, kWideHeads = 128;
constexpr int kQPitch = kE + 8;                              // query row pitch in LDS (elements)
constexpr int kRowBytes = kE * 2, kRowChunks = kE / 8, kTileBytes = kTile * kRowBytes;
constexpr int kTileLoads = kTile * kRowChunks / 64;          // 64-lane loads per tile (36)
static_assert(kTileLoads % kWideWaves == 0, "whole loads per wave");

// byte offset of chunk c of row r in a tile
__device__ __forceinline__ int tile_off(int r, int c) {
  return 1024 * (c >> 1) + 512 * (c & 1) + 16 * ((r + 8 * (c & 1)) & 31);
}

typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s_t lds_v4s_t;

__device__ __forceinline__ uint2 lds_read_tr(const char* p) {
  const v4s_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t*)p);
  return __builtin_bit_cast(uint2, r);
}

struct WideShared {
  __attribute__((aligned(16))) char kbuf[2][kTileBytes];
  // queries of each wave's second head block (the first stays in registers)
  __attribute__((aligned(16))) bf16_t qs[kWideWaves][16][kQPitch];
  const char* row_ptr[3][kTile];
  uint32_t row_mask[3];                                      // bit r: row r of the tile present
  int flag[2][kWideWaves];
};

// One block's split.  EXACT = false: the main pass; returns true, without
// writing anything, when a logit left its head's reference band.  EXACT =
// true: the split again, first for each head's exact maximum, then
// accumulating against it, one tile at a time.
template <bool EXACT>
__device__ __forceinline__ bool wide_split(const AttnArgs& a, WideShared& sh) {
  auto& kbuf = sh.kbuf;
  auto& qs = sh.qs;
  auto& row_ptr = sh.row_ptr;
  auto& row_mask = sh.row_mask;
  auto& flag = sh.flag;
  // uniform scalars the loop uses, pinned to scalar registers
  const float c_log2 = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, a.c)));

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int split = blockIdx.x, hg = blockIdx.y, b = blockIdx.z;
  const int col = lane & 15, g = lane >> 4;
  int hh[2];
  bool hok[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    hh[j] = hg * kWideHeads + wave * 32 + j * 16 + col;
    hok[j] = hh[j] < a.H;
  }
  const bf16_t* q = reinterpret_cast<const bf16_t*>(a.q);
  const char* ent = reinterpret_cast<const char*>(a.entries);
  const char* win = reinterpret_cast<const char*>(a.window);
  const char* safe_row = reinterpret_cast<const char*>(q + (int64_t)b * a.H * kE);

  // query fragments of head block 0: k-slots (g, t) <-> dim 32 ks + 8g + t
  Frag<bf16_t> qf[18];
  {
    const bf16_t* qp = q + ((int64_t)b * a.H + (hok[0] ? hh[0] : 0)) * kE + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      frag_load(qf[ks], qp + 32 * ks);
      if (!hok[0]) qf[ks].v = u32x4{0u, 0u, 0u, 0u};
    }
  }
  // head block 1 to LDS: lane (col, g) copies dims 8g..8g+7 of every 32
  {
    const bf16_t* qp = q + ((int64_t)b * a.H + (hok[1] ? hh[1] : 0)) * kE + 8 * g;
#pragma unroll 6
    for (int ks = 0; ks < 18; ++ks) {
      uint4 v = *reinterpret_cast<const uint4*>(qp + 32 * ks);
      if (!hok[1]) v = make_uint4(0u, 0u, 0u, 0u);
      *reinterpret_cast<uint4*>(&qs[wave][col][32 * ks + 8 * g]) = v;
    }
  }

  f32x4 O[2][32];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int db = 0; db < 32; ++db) O[j][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};

  int64_t win_row0 = 0;
  int nwin = a.W;
  if (a.q_pos) {
    const int64_t pos = a.q_pos[b];
    int64_t lo = pos - a.W + 1;
    if (lo < 0) lo = 0;
    nwin = (int)(pos - lo + 1);
    win_row0 = lo - a.win_pos0;
  }
  const int s_begin = split * a.slots_per_split;
  const int s_end = min(a.nslots, s_begin + a.slots_per_split);
  const int ntiles = s_end > s_begin ? (s_end - s_begin + kTile - 1) / kTile : 0;

  // Row addresses of tile t into ring slot t % 3 (wave 0, one lane per row).
  // A selected entry comes in as e_sel, loaded a tile ahead by sel_load.
  auto sel_load = [&](int t) {
    int e = -1;
    if (threadIdx.x < kTile && !a.dense) {
      const int s = s_begin + t * kTile + threadIdx.x;
      if (s < s_end && s < a.k) e = a.idx[(int64_t)b * a.k + s];
    }
    return e;
  };
  auto resolve = [&](int t, int e_sel) {
    int ok_lane = 0;
    if (threadIdx.x < kTile) {
      const int s = s_begin + t * kTile + threadIdx.x;
      const char* p = safe_row;
      int ok = 0;
      if (s < s_end) {
        if (a.dense) {
          ok = 1;
          p = ent + ((int64_t)b * a.ent_bstride + (int64_t)s * kE) * 2;
        } else if (s < a.k) {
          ok = (e_sel >= 0 && e_sel < a.N);                    // -1 (or out of range): no row
          if (ok) p = ent + ((int64_t)b * a.ent_bstride + (int64_t)e_sel * kE) * 2;
        } else {
          const int w = s - a.k;
          const int64_t r = win_row0 + w;
          ok = w < nwin && r >= 0 && r < a.win_rows;           // rows outside the buffer are skipped
          if (ok) p = win + ((int64_t)b * a.win_bstride + r * kE) * 2;
        }
      }
      row_ptr[t % 3][threadIdx.x] = p;
      ok_lane = ok;
    }
    if (threadIdx.x < 64) {                                  // wave 0: bit r = row r present
      const uint64_t m = __ballot(threadIdx.x < kTile && ok_lane);
      if (threadIdx.x == 0) row_mask[t % 3] = (uint32_t)m;
    }
  };
  // gather tile t into buffer k: copy n (64 lanes x 16 bytes) fills LDS bytes
  // [1024 n, 1024 n + 1024) of the buffer with chunks 2n (lanes 0..31) and
  // 2n + 1 (lanes 32..63); a lane's copies all come from one row
  auto issue = [&](int t, int k) {
    const unsigned base = lds_offset(kbuf[k]);
    const int par = lane >> 5;
    const int r = ((lane & 31) - 8 * par) & 31;
    const char* rowp = row_ptr[t % 3][r] + 16 * par;
#pragma unroll
    for (int i = 0; i < kTileLoads / kWideWaves; ++i) {
      const int n = wave + i * kWideWaves;
      dma16(rowp + 32 * n, (unsigned)__builtin_amdgcn_readfirstlane(base + 1024 * n));
    }
  };

  // Lane offsets of the LDS read patterns, derived from the lane id each
  // time a tile starts: nothing lane-dependent stays in a register across
  // the loop.
  struct LaneOffs {
    int k0, k1;        // logit rows col and 16 + col at chunk g (+ 2048 per 32-dim step)
    int v0, v1;        // value rows 4g + col/4 and 16 + that (+ 1024 per 16-dim block)
    int qoff;          // second head block's queries in LDS
    int g4;            // 4 g
  };
  auto lane_offs = [&]() {
    int lid;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lid));
    const int c = lid & 15, gg = lid >> 4;
    LaneOffs o;
    o.k0 = tile_off(c, gg);
    o.k1 = tile_off(16 + c, gg);
    const int vr = 4 * gg + (c >> 2), vc = (c & 3) >> 1;     // chunk 2 db + vc, half c & 1
    o.v0 = tile_off(vr, vc) + ((c & 1) << 3);
    o.v1 = tile_off(16 + vr, vc) + ((c & 1) << 3);
    o.qoff = (int)lds_offset(&qs[wave][c][8 * gg]);
    o.g4 = 4 * gg;
    return o;
  };

  int flagged_here = 0;
  // logits S^T[row, head] of one tile: rows 0..15 in S0, 16..31 in S1
  auto qk_tile = [&](const char* kb, const LaneOffs& L, f32x4* S0, f32x4* S1) {
#pragma unroll
    for (int j = 0; j < 2; ++j) { S0[j] = f32x4{0.f, 0.f, 0.f, 0.f}; S1[j] = S0[j]; }
    // fragments of step ks: rows col and 16 + col at chunk 4 ks + g, and the
    // second head block's queries; double-buffered one step ahead
    Frag<bf16_t> A0[2], A1[2], Q1[2];
    auto kfrag = [&](int ks, int u) {
      const uint4 x0 = *reinterpret_cast<const uint4*>(kb + L.k0 + 2048 * ks);
      const uint4 x1 = *reinterpret_cast<const uint4*>(kb + L.k1 + 2048 * ks);
      const u32x4 y = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
          (const __attribute__((address_space(3))) char*)(uintptr_t)(L.qoff + 64 * ks));
      A0[u].v = u32x4{x0.x, x0.y, x0.z, x0.w};
      A1[u].v = u32x4{x1.x, x1.y, x1.z, x1.w};
      Q1[u].v = y;
    };
    kfrag(0, 0);
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      const int u = ks & 1;
      if (ks + 1 < 18) kfrag(ks + 1, u ^ 1);
      fence_sched();
      mma16(S0[0], A0[u], qf[ks]);
      mma16(S1[0], A1[u], qf[ks]);
      mma16(S0[1], A0[u], Q1[u]);
      mma16(S1[1], A1[u], Q1[u]);
    }
  };
  // masked, scaled logits of one head block (log2 units) and their tile max
  auto tile_logits = [&](int t, const LaneOffs& L, const f32x4& s0, const f32x4& s1, float* sv) {
    const uint32_t m = row_mask[t % 3] >> L.g4;               // rows 4g + i and 16 + 4g + i
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float x = i < 4 ? s0[i] : s1[i - 4];
      const int bit = i < 4 ? i : 12 + i;
      sv[i] = ((m >> bit) & 1u) ? x * c_log2 : -INFINITY;
      tmax = fmaxf(tmax, sv[i]);
    }
    return max_xor32(max_xor16(tmax));
  };
  // one tile of the accumulation (check: the main pass, which sets the
  // references and flags logits past the band)
  auto tile_body = [&](int t, const char* kb, bool check) {
    const LaneOffs L = lane_offs();
    f32x4 S0[2], S1[2];
    qk_tile(kb, L, S0, S1);
    Frag<bf16_t> pf[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float sv[8];
      const float tmax = tile_logits(t, L, S0[j], S1[j], sv);
      if (check) {
        if (m_ref[j] == -INFINITY) m_ref[j] = tmax;
        else if (tmax > m_ref[j] + kRefBand) flagged_here = 1;
      }
      const float m_use = (m_ref[j] == -INFINITY) ? 0.f : m_ref[j];
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        sv[i] = __builtin_amdgcn_exp2f(sv[i] - m_use);
        psum += sv[i];
      }
      l_run[j] += psum;
      p_frag(pf[j], sv);
    }
    // O^T[d, head] += V^T[d, rows] . P^T[rows, head]; value fragments of
    // 16-dim block db (chunks 2 db, 2 db + 1) run three blocks ahead
    Frag<bf16_t> VF[4];
    auto vfrag = [&](int db) {
      const uint2 v0 = lds_read_tr(kb + L.v0 + 1024 * db), v1 = lds_read_tr(kb + L.v1 + 1024 * db);
      VF[db & 3].v = u32x4{v0.x, v0.y, v1.x, v1.y};
    };
    vfrag(0);
    vfrag(1);
    vfrag(2);
#pragma unroll
    for (int db = 0; db < 32; ++db) {
      if (db + 3 < 32) vfrag(db + 3);
      fence_sched();
#pragma unroll
      for (int j = 0; j < 2; ++j) mma16(O[j][db], VF[db & 3], pf[j]);
    }
  };
  auto any_flag = [&](int t) {
    int any = 0;
#pragma unroll
    for (int w = 0; w < kWideWaves; ++w) any |= flag[t & 1][w];
    return any != 0;
  };

  // prologue: rows of tiles 0 and 1, selection of tile 2, tile 0 in flight
  int e_next = -1;
  if (ntiles > 0) resolve(0, sel_load(0));
  if (ntiles > 1) resolve(1, sel_load(1));
  if (ntiles > 2) e_next = sel_load(2);
  __syncthreads();                                           // rows and queries in LDS
  if (ntiles > 0) issue(0, 0);

  if constexpr (!EXACT) {
    bool redo = false;
    for (int t = 0; t < ntiles; ++t) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();                                       // tile t landed; tile t-1 fully read
      if (t > 0 && any_flag(t - 1)) { redo = true; break; }  // block-uniform
      // every load but the gather is issued first: a wait for it would
      // otherwise drain the gather too
      if (t + 2 < ntiles) resolve(t + 2, e_next);
      if (t + 3 < ntiles) e_next = sel_load(t + 3);
      if (t + 1 < ntiles) issue(t + 1, (t + 1) & 1);
      tile_body(t, kbuf[t & 1], true);
      const int wave_flag = __any(flagged_here);             // any head of this wave
      if (lane == 0) flag[t & 1][wave] = wave_flag;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (!redo && ntiles > 0) redo = any_flag(ntiles - 1);
    if (redo) return true;
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    auto load_tile = [&](int t) {
      __syncthreads();                                       // buffer and ring free
      resolve(t, sel_load(t));
      __syncthreads();
      issue(t, 0);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    };
    float mx[2] = {-INFINITY, -INFINITY};
    for (int t = 0; t < ntiles; ++t) {
      load_tile(t);
      const LaneOffs L = lane_offs();
      f32x4 S0[2], S1[2];
      qk_tile(kbuf[0], L, S0, S1);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float sv[8];
        mx[j] = fmaxf(mx[j], tile_logits(t, L, S0[j], S1[j], sv));
      }
    }
    m_ref[0] = mx[0];
    m_ref[1] = mx[1];
    for (int t = 0; t < ntiles; ++t) {
      load_tile(t);
      tile_body(t, kbuf[0], false);
    }
  }

  const float LN2 = 0.6931471805599453f;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const float l = sum_xor32(sum_xor16(l_run[j]));
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const float lse2 = l > 0.f ? m_ref[j] + __log2f(l) : -INFINITY;
    if (!hok[j]) continue;
    const int h = hh[j];
    if (a.nsplit == 1) {
      bf16_t* o = reinterpret_cast<bf16_t*>(a.out) + ((int64_t)b * a.H + h) * kDv;
#pragma unroll
      for (int db = 0; db < 32; ++db)
        store_out4<bf16_t>(o + 16 * db + 4 * g, O[j][db][0] * inv, O[j][db][1] * inv,
                           O[j][db][2] * inv, O[j][db][3] * inv);
      if (a.lse && g == 0) a.lse[(int64_t)b * a.H + h] = lse2 * LN2;
    } else {
      float* o = a.o_part + (((int64_t)b * a.H + h) * a.nsplit + split) * kDv;
#pragma unroll
      for (int db = 0; db < 32; ++db)
        store_out4<float>(o + 16 * db + 4 * g, O[j][db][0] * inv, O[j][db][1] * inv,
                          O[j][db][2] * inv, O[j][db][3] * inv);
      if (g == 0) a.lse_part[((int64_t)b * a.H + h) * a.nsplit + split] = lse2 * LN2;
    }
  }
  return false;
}

__device__ __noinline__ void wide_split_exact(const AttnArgs& a, WideShared& sh) {
  wide_split<true>(a, sh);
}

__global__ __launch_bounds__(64 * kWideWaves) void attend_wide_kernel(AttnArgs a) {
  __shared__ WideShared sh;
  __shared__ AttnArgs args;
  if (wide_split<false>(a, sh)) {                            // rare
    // the arguments reach the out-of-line pass through LDS, so that the
    // main pass never needs an addressable copy of them
    if (threadIdx.x == 0) args = a;
    __syncthreads();
    wide_split_exact(args, sh);
  }
}

// One wave per (query, head): lse = ln sum_s exp(lse_s); out = sum_s
// exp(lse_s - lse) o_s.  Splits are combined in index order.
template <class T>
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ o_part,
                                                    const float* __restrict__ lse_part, int64_t BH,
                                                    int S, T* __restrict__ out,
                                                    float* __restrict__ lse) {
  const int lane = threadIdx.x & 63;
  const int64_t bh = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (bh >= BH) return;
  const float* lp = lse_part + bh * S;
  float mx = -INFINITY;
  for (int s = 0; s < S; ++s) mx = fmaxf(mx, lp[s]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float tot = 0.f;
  if (mx != -INFINITY) {
    for (int s = 0; s < S; ++s) {
      const float w = __expf(lp[s] - mx);
      tot += w;
      float v[8];
      Row8<float>::load(o_part + (bh * S + s) * kDv + lane * 8, v);
#pragma unroll
      for (int d = 0; d < 8; ++d) acc[d] = fmaf(w, v[d], acc[d]);
    }
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
#pragma unroll
  for (int d = 0; d < 8; ++d) acc[d] *= inv;
  Row8<T>::store(out + bh * kDv + lane * 8, acc);
  if (lse && lane == 0) lse[bh] = tot > 0.f ? mx + __logf(tot) : -INFINITY;
}

// ------------------------------------------------------------------ host

int attend_heads_per_block(int dt, int H) {
  (void)H;
  return dt == 0 ? 16 * AttnCfg<float>::NW : kWideHeads;
}

int attend_splits(int dt, int64_t B, int H, int64_t nslots) {
  const int hpb = attend_heads_per_block(dt, H);
  const int64_t blocks = B * ((H + hpb - 1) / hpb);
  const int64_t tiles = (nslots + kTile - 1) / kTile;
  if (tiles == 0) return 1;
  // about one round of resident blocks (the bf16 kernel holds one block per
  // compute unit): more splits than that only add partial outputs
  const int64_t target = dt == 0 ? 512 : 256;
  int64_t s = (target + blocks - 1) / blocks;
  const int64_t cap = tiles / 2 > 1 ? tiles / 2 : 1;
  if (s > cap) s = cap;
  if (s > 64) s = 64;
  if (s < 1) s = 1;
  // equal whole tiles per split; drop splits that would be empty
  const int64_t per = (tiles + s - 1) / s;
  return (int)((tiles + per - 1) / per);
}

size_t attend_partial_bytes(int dt, int64_t B, int H, int64_t nslots) {
  const int S = attend_splits(dt, B, H, nslots);
  if (S <= 1) return 0;
  return (size_t)B * H * S * (kDv + 1) * sizeof(float) + 256;
}

template <class T>
static hipError_t launch_attend_t(const AttendParams& p, void* ws, hipStream_t stream) {
  typedef AttnCfg<T> C;
  (void)sizeof(C);
  AttnArgs a;
  a.q = p.q; a.entries = p.entries; a.window = p.window; a.idx = p.idx; a.q_pos = p.q_pos;
  a.ent_bstride = p.ent_bstride; a.win_bstride = p.win_bstride; a.win_pos0 = p.win_pos0;
  a.win_rows = p.win_rows; a.dense = p.dense;
  a.N = p.N; a.B = (int)p.B; a.H = p.H; a.W = p.dense ? 0 : p.W; a.k = p.dense ? 0 : p.k;
  a.nslots = (int)(p.dense ? p.N : (int64_t)p.k + p.W);
  a.c = p.scale * 1.4426950408889634f;
  a.out = p.out; a.lse = p.lse;
  const int S = attend_splits(p.dt, p.B, p.H, a.nslots);
  const int64_t tiles = (a.nslots + kTile - 1) / kTile;
  a.nsplit = S;
  a.slots_per_split = (int)(((tiles + S - 1) / S) * kTile);
  a.o_part = (float*)ws;
  a.lse_part = a.o_part + (size_t)p.B * p.H * S * kDv;
  const int hpb = attend_heads_per_block(p.dt, p.H);
  dim3 grid(S, (p.H + hpb - 1) / hpb, (unsigned)p.B);
  if constexpr (sizeof(T) == 2)
    hipLaunchKernelGGL(attend_wide_kernel, grid, dim3(64 * kWideWaves), 0, stream, a);
  else
    hipLaunchKernelGGL((attend_kernel<T, 1>), grid, dim3(64 * C::NW), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S == 1) return e;
  const int64_t BH = p.B * p.H;
  hipLaunchKernelGGL(merge_kernel<T>, dim3((unsigned)((BH + 3) / 4)), dim3(256), 0, stream,
                     a.o_part, a.lse_part, BH, S, (T*)p.out, p.lse);
  return hipGetLastError();
}

hipError_t launch_attend(const AttendParams& p, void* ws, hipStream_t stream) {
  if (p.dt == 0) return launch_attend_t<float>(p, ws, stream);
  return launch_attend_t<bf16_t>(p, ws, stream);
}

hipError_t launch_merge(int dt, const float* o_part, const float* lse_part, int64_t BH, int S,
                        void* out, float* lse, hipStream_t stream) {
  if (dt == 0)
    hipLaunchKernelGGL(merge_kernel<float>, dim3((unsigned)((BH + 3) / 4)), dim3(256), 0, stream,
                       o_part, lse_part, BH, S, (float*)out, lse);
  else
    hipLaunchKernelGGL(merge_kernel<bf16_t>, dim3((unsigned)((BH + 3) / 4)), dim3(256), 0, stream,
                       o_part, lse_part, BH, S, (bf16_t*)out, lse);
  return hipGetLastError();
}

}  // namespace cskv
