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
// weighted sum).  Each wave owns MN heads (MN = 32 with the bf16 32x32x16
// MFMA, MN = 16 with the fp32 16x16x4 MFMA) and keeps their queries and
// output accumulators in registers.  Per tile:
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

template <class T> struct AttnCfg;
template <> struct AttnCfg<bf16_t> {
  static constexpr int MN = 16, NW = 4;                      // 64 heads per block
  static constexpr int EPC = 8;                              // elements per 16-byte chunk
  static constexpr int KP = kE + 8;                          // K tile row pitch (elements)
  static constexpr int VP = kTile + 4;                       // V^T row pitch (elements)
};
template <> struct AttnCfg<float> {
  static constexpr int MN = 16, NW = 1;                      // 16 heads per block
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

// Number of accumulator values per lane of one MN x MN output tile.
template <int MN> struct Acc;
template <> struct Acc<32> { typedef f32x16 type; static constexpr int n = 16; };
template <> struct Acc<16> { typedef f32x4 type; static constexpr int n = 4; };

// Row (within a 32-row tile) held by accumulator value i of lane group g of
// the logits product.  MN = 32: one 32x32 tile; MN = 16: two 16-row tiles
// stacked (values 0..3 in the first, 4..7 in the second).
template <int MN> __device__ __forceinline__ int srow(int g, int i);
template <> __device__ __forceinline__ int srow<32>(int g, int i) { return 8 * (i >> 2) + 4 * g + (i & 3); }
template <> __device__ __forceinline__ int srow<16>(int g, int i) { return 16 * (i >> 2) + 4 * g + (i & 3); }

template <class T>
__global__ __launch_bounds__(64 * AttnCfg<T>::NW) void attend_kernel(AttnArgs a) {
  typedef AttnCfg<T> C;
  constexpr int MN = C::MN, NW = C::NW, NT = 64 * NW;
  constexpr int NS = (MN == 32) ? 16 : 8;                    // logits per lane per tile
  constexpr int KSTEP = (MN == 32) ? 16 : 32;                // contraction per MFMA step
  constexpr int NKS = kE / KSTEP;
  constexpr int NDB = kDv / MN;                              // output d-blocks
  __shared__ __attribute__((aligned(16))) T Ks[kTile * C::KP];
  __shared__ __attribute__((aligned(16))) T Vt[kDv * C::VP];
  __shared__ int64_t row_off[2][kTile];
  __shared__ int row_ok[2][kTile];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int split = blockIdx.x, hg = blockIdx.y, b = blockIdx.z;
  const int col = lane % MN, g = lane / MN;
  const int h = (hg * NW + wave) * MN + col;
  const bool h_ok = h < a.H;
  const T* q = reinterpret_cast<const T*>(a.q);
  const T* ent = reinterpret_cast<const T*>(a.entries);
  const T* win = reinterpret_cast<const T*>(a.window);

  // query fragments for this lane's head: k-slots (g, t) <-> dim KSTEP*ks + 8g + t
  Frag<T> qf[NKS];
  {
    const T* qp = q + ((int64_t)b * a.H + (h_ok ? h : 0)) * kE;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      frag_load(qf[ks], qp + ks * KSTEP + 8 * g);
      if (!h_ok) {
        Frag<T> z{};
        qf[ks] = z;
      }
    }
  }
  typename Acc<MN>::type O[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < Acc<MN>::n; ++i) O[db][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

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
    // logits S^T[row, head]
    float sv[NS];
    if constexpr (MN == 32) {
      f32x16 S;
#pragma unroll
      for (int i = 0; i < 16; ++i) S[i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        Frag<T> af;
        frag_load(af, Ks + col * C::KP + ks * KSTEP + 8 * g);
        mma32(S, af, qf[ks]);
        if ((ks & 3) == 3) fence_sched();
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) sv[i] = S[i];
    } else {
      f32x4 S0, S1;
#pragma unroll
      for (int i = 0; i < 4; ++i) { S0[i] = 0.f; S1[i] = 0.f; }
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        Frag<T> a0, a1;
        frag_load(a0, Ks + col * C::KP + ks * KSTEP + 8 * g);
        frag_load(a1, Ks + (16 + col) * C::KP + ks * KSTEP + 8 * g);
        mma16(S0, a0, qf[ks]);
        mma16(S1, a1, qf[ks]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) { sv[i] = S0[i]; sv[4 + i] = S1[i]; }
    }
    // online softmax (per head = per lane column)
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int r = srow<MN>(g, i);
      sv[i] = tile_ok[r] ? sv[i] * a.c : -INFINITY;
      tmax = fmaxf(tmax, sv[i]);
    }
    if constexpr (MN == 32) {
      tmax = fmaxf(tmax, shfl_xor(tmax, 32));
    } else {
      tmax = fmaxf(tmax, shfl_xor(tmax, 16));
      tmax = fmaxf(tmax, shfl_xor(tmax, 32));
    }
    // Lazy rescaling: the reference max of a head only moves when the tile
    // max exceeds it by more than kLazy (log2 units), so weights stay below
    // 2^kLazy and the accumulators are rescaled rarely (wave-uniform branch).
    if (__any(tmax > m_run + kLazy)) {
      const float m_new = fmaxf(m_run, tmax);
      const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < Acc<MN>::n; ++i) O[db][i] *= alpha;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      sv[i] = __builtin_amdgcn_exp2f(sv[i] - m_use);
      psum += sv[i];
    }
    l_run += psum;

    // O^T[d, head] += V^T[d, rows] . P^T[rows, head]
    if constexpr (MN == 32) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        Frag<T> pf;
        p_frag(pf, sv + 8 * st);
        const int r0 = 16 * st + 4 * g, r1 = r0 + 8;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          Frag<T> vf;
          vt_frag(vf, Vt + (db * MN + col) * C::VP, r0, r1);
          mma32(O[db], vf, pf);
          if ((db & 3) == 3) fence_sched();
        }
      }
    } else {
      Frag<T> pf;
      p_frag(pf, sv);
      const int r0 = 4 * g, r1 = 16 + 4 * g;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        Frag<T> vf;
        vt_frag(vf, Vt + (db * MN + col) * C::VP, r0, r1);
        mma16(O[db], vf, pf);
      }
    }
    __syncthreads();
    if constexpr (kOverlap) slot ^= 1;
  }

  // finish: total row sum of this head over the lane groups
  if constexpr (MN == 32) {
    l_run += shfl_xor(l_run, 32);
  } else {
    l_run += shfl_xor(l_run, 16);
    l_run += shfl_xor(l_run, 32);
  }
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  const float lse2 = l_run > 0.f ? m_run + __log2f(l_run) : -INFINITY;
  const float LN2 = 0.6931471805599453f;
  if (!h_ok) return;
  if (a.nsplit == 1) {
    T* o = reinterpret_cast<T*>(a.out) + ((int64_t)b * a.H + h) * kDv;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int j = 0; j < Acc<MN>::n / 4; ++j) {
        const int d = db * MN + (MN == 32 ? 8 * j : 0) + 4 * g;
        store_out4<T>(o + d, O[db][4 * j] * inv, O[db][4 * j + 1] * inv, O[db][4 * j + 2] * inv,
                      O[db][4 * j + 3] * inv);
      }
    }
    if (a.lse && g == 0) a.lse[(int64_t)b * a.H + h] = lse2 * LN2;
  } else {
    float* o = a.o_part + (((int64_t)b * a.H + h) * a.nsplit + split) * kDv;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int j = 0; j < Acc<MN>::n / 4; ++j) {
        const int d = db * MN + (MN == 32 ? 8 * j : 0) + 4 * g;
        store_out4<float>(o + d, O[db][4 * j] * inv, O[db][4 * j + 1] * inv,
                          O[db][4 * j + 2] * inv, O[db][4 * j + 3] * inv);
      }
    }
    if (g == 0) a.lse_part[((int64_t)b * a.H + h) * a.nsplit + split] = lse2 * LN2;
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

int attend_heads_per_block(int dt) { return dt == 0 ? 16 : 64; }

int attend_splits(int dt, int64_t B, int H, int64_t nslots) {
  const int hpb = attend_heads_per_block(dt);
  const int64_t blocks = B * ((H + hpb - 1) / hpb);
  const int64_t tiles = (nslots + kTile - 1) / kTile;
  if (tiles == 0) return 1;
  int64_t s = (512 + blocks - 1) / blocks;
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
  const int hpb = C::MN * C::NW;
  dim3 grid(S, (p.H + hpb - 1) / hpb, (unsigned)p.B);
  hipLaunchKernelGGL(attend_kernel<T>, grid, dim3(64 * C::NW), 0, stream, a);
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
