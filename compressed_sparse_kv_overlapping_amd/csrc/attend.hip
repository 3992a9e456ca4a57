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
// that query's rows, in tiles of 32 rows.  Two kernels: attend_wide_kernel
// (bf16, 128 heads per block, described at its section below) and
// attend_kernel (fp32, 16 heads per block), which gathers each tile into LDS
// twice, row-major (K, for the logits) and transposed (V^T, for the weighted
// sum), with 16x16x4 fp32 MFMA; each wave keeps its heads' queries and
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
#include "fp4.hpp"
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
  static constexpr int NW = 4;                               // 64 heads per block
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
  int hm;                    // dense with q_pos: entry i visible iff (i+1)*hm <= q_pos[b]+1
  const float* sink;         // [H] attention-sink logits (nullable), applied where splits end
  float norm_eps;            // query / entry normalisation epsilon (kernels instantiated for it)
  int B, H, W, k, nslots, slots_per_split, nsplit;
  float c;                   // scale * log2(e)
  void* out;                 // [B][H][512] when nsplit == 1
  float* lse;                // [B][H] (nullable)
  float* o_part;             // [B][H][nsplit][512]
  float* lse_part;           // [B][H][nsplit]
};

// Final normalisation of one head.  l: the sum of its weights relative to
// the reference m2 (log2 units); s2: its attention-sink logit in log2 units
// (-inf: no sink), one more softmax term with a zero value.  *scale
// multiplies the accumulators; *lse2 is log2 of the whole denominator.
__device__ __forceinline__ void head_norm(float l, float m2, float s2, float* scale, float* lse2) {
  if (s2 == -INFINITY) {
    *scale = l > 0.f ? 1.f / l : 0.f;
    *lse2 = l > 0.f ? m2 + __log2f(l) : -INFINITY;
    return;
  }
  const float M = l > 0.f ? fmaxf(m2, s2) : s2;
  const float w = l > 0.f ? __builtin_amdgcn_exp2f(m2 - M) : 0.f;
  const float den = l * w + __builtin_amdgcn_exp2f(s2 - M);
  *scale = w / den;
  *lse2 = M + __log2f(den);
}

// End of a split's rows: in dense mode at a prefill chunk, the entries the
// query at q_pos[b] sees (i with (i+1)*hm <= q_pos[b]+1) end the range, so
// tiles past them are not visited at all.
__device__ __forceinline__ int dense_end(const AttnArgs& a, int b, int s_begin, int s_end) {
  if (!a.dense || a.hm <= 0 || !a.q_pos) return s_end;
  const int64_t p1 = a.q_pos[b] + 1;
  const int64_t vis = p1 > 0 ? p1 / a.hm : 0;
  return vis < s_end ? (vis > s_begin ? (int)vis : s_begin) : s_end;
}

// Block order over the XCDs: the dispatcher deals linear block ids round-
// robin over the 8 XCDs; logical block L = xcd_block(id, G) gives each XCD a
// contiguous range of logical blocks, so the splits of one query (and, with
// the same order in the merge, that query's merge blocks) share one XCD.
__device__ __forceinline__ int xcd_block(int id, int G) {
  const int q = G / 8, rem = G % 8;
  const int x = id % 8, slot = id / 8;
  return x * q + (x < rem ? x : rem) + slot;
}

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
// from LDS feeds two MFMAs, which halves the LDS traffic per flop.  NORM:
// queries and compressed entries normalised to unit root-mean-square (as in
// the wide kernel below; the tile's row factors are computed from its
// staged rows, two lanes a row).
template <class T, int HB, bool NORM>
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
  __shared__ float row_g[kTile];                             // row factors (NORM)

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
  // each head's softmax scale, with its query's factor (NORM): a head's 576
  // dims are spread over the lanes col, col+16, col+32, col+48
  float c_h[HB];
#pragma unroll
  for (int j = 0; j < HB; ++j) {
    c_h[j] = a.c;
    if constexpr (NORM) {
      float ss = 0.f;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int t = 0; t < 8; ++t) ss = fmaf((float)qf[j][ks].v[t], (float)qf[j][ks].v[t], ss);
      ss += shfl_xor(ss, 16);
      ss += shfl_xor(ss, 32);
      c_h[j] = a.c * __frsqrt_rn(ss * (1.f / kE) + a.norm_eps);
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
  const int s_end = dense_end(a, b, s_begin, min(a.nslots, s_begin + a.slots_per_split));

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
    if constexpr (NORM) {
      // row factor of row r: threads 2r and 2r+1 sum the squares of its two
      // halves; 1 for raw window rows
      for (int r0 = 0; r0 < kTile; r0 += NT / 2) {
        const int r = r0 + threadIdx.x / 2, h = threadIdx.x & 1;
        float ss = 0.f;
        if (r < kTile) {
          const T* rp = Ks + r * C::KP + h * (kE / 2);
          for (int e = 0; e < kE / 2; ++e) ss = fmaf((float)rp[e], (float)rp[e], ss);
        }
        ss += __shfl_xor(ss, 1, 64);
        const int sl = t0 + r;
        // absent rows (zero-filled) take 1, so that their zero weight stays 0
        if (r < kTile && h == 0)
          row_g[r] = (tile_ok[r] && (a.dense || sl < a.k)) ? __frsqrt_rn(ss * (1.f / kE) + a.norm_eps)
                                                           : 1.f;
      }
      __syncthreads();
    }
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
        const float c = NORM ? c_h[j] * row_g[srow(g, i)] : a.c;
        sv[i] = tile_ok[srow(g, i)] ? sv[i] * c : -INFINITY;
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
      if constexpr (NORM) {
        // the weighted sum takes the normalised rows; the sum above does not
#pragma unroll
        for (int i = 0; i < 8; ++i) sv[i] *= row_g[srow(g, i)];
      }
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
    // the sink joins where the splits end: here with one split, else in
    // the merge
    const float s2 = (a.sink && a.nsplit == 1) ? a.sink[hok[j] ? hh[j] : 0] * 1.4426950408889634f
                                               : -INFINITY;
    float inv, lse2;
    head_norm(l, m_run[j], s2, &inv, &lse2);
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
// each wave owns 32 heads and keeps their queries (144 registers) and their
// output accumulators (O^T: 512 dims x 32 heads, 256 registers) for the
// whole split.  One wave per SIMD.  Both products use the 32x32x16 bf16
// MFMA:
//   S^T[32 rows, 32 heads]  = K_tile . Q^T        36 k-steps, A = keys (LDS)
//   O^T[32 dims, 32 heads] += V^T_tile . P^T      16 dim blocks x 2 k-steps,
//                                                 A = values (LDS, transposed)
// Lane l of S^T holds head l % 32 and the 16 rows 8 q + 4 (l / 32) + i
// (register 4 q + i).  Rounded to bf16, registers 8u..8u+7 are the B operand
// of k-step u of the second product as they stand: slot t there stands for
// row 16 u + 4 (l / 32) + 8 (t / 4) + t % 4, and the value fragment of the
// lane reads those same rows (two 4-row transposed reads).
//
// The loop is software-pipelined: while the MFMAs of the logits of tile t+1
// run, the softmax of tile t (VALU work) is issued between them, one short
// piece per k-step; the weighted sum of tile t follows.  Tiles are gathered
// from HBM straight into LDS (global_load_lds, 16 bytes per lane, no
// registers) into three buffers: tile t is read for its values, tile t+1 for
// its keys, tile t+2 is in flight.
//
// Tile layout: 32 rows x 72 chunks of 16 bytes, row-major (1152 bytes a
// row); chunk c of row r sits in slot c ^ g(r) of the row, with
//   g(r) = 4 ((r / 2) % 2) + (r / 4) % 4,
// a permutation inside each aligned group of 8 chunks (128 bytes).  Read
// patterns (64 banks of 4 bytes; a 16-byte slot covers 4 banks and slot s of
// row r the bank group (8 r + s) % 16):
//   keys:   per 16 lanes, 16 rows of one chunk (ds_read_b128): the 8 even
//           rows take the 8 values of g, the 8 odd rows the same 8 shifted
//           by 8 groups: every bank once;
//   values: per 32 lanes, 4 rows 4m..4m+3 of the 4 chunks of a 32-dim block
//           (ds_read_b64_tr_b16): rows 4m and 4m+2 take opposite halves of
//           the 8 groups (bit 2 of g differs), 4m+1 and 4m+3 the same shifted
//           by 8: every bank once.
// Copy n of a tile fills slots [64 n, 64 n + 64) of the row-major image:
// lane i takes slot q = 64 n + i, i.e. row q / 72, chunk (q % 72) ^ g(row),
// so one copy reads at most two rows' contiguous bytes (about 9 cache lines
// instead of one per lane).  The copies are issued from inline assembly, so
// the compiler does not see an LDS write in flight; the loop waits for them
// explicitly before the barrier that opens each tile.  In the pipelined loop
// a wave issues its 9 copies of tile t+2 spread over the logit steps of tile
// t+1.
//
// Softmax reference: a head's first visible tile sets it (its accumulators
// are still zero then) and it never moves, so the accumulators are never
// rescaled in the loop; later weights may reach 2^kRefBand, far inside fp32
// and bf16 range.  A logit beyond that band is flagged, and the block then
// runs the split again: first for each head's exact maximum, then
// accumulating against it.
constexpr int kWideWaves = 4, kWideHeads = 128;
constexpr int kRowBytes = kE * 2, kTileBytes = kTile * kRowBytes;
constexpr int kTileLoads = kTile * (kE / 8) / 64;            // 64-lane copies per tile (36)
constexpr int kQSteps = kE / 16;                             // k-steps of the logits (36)
constexpr int kVBlocks = kDv / 32;                           // 32-dim blocks of the values (16)
constexpr int kBufs = 3, kRing = 4;
constexpr int kKDepth = 4, kVDepth = 4;                      // LDS fragment prefetch depths
constexpr int kCopies = kTileLoads / kWideWaves;             // copies per wave per tile (9)
static_assert(kTileLoads % kWideWaves == 0, "whole copies per wave");
static_assert(kCopies * 4 <= kQSteps, "a wave's copies fit between the logit steps");

// slot permutation of row r, and the byte offset of chunk c of row r
__device__ __forceinline__ int row_swz(int r) { return 4 * ((r >> 1) & 1) + ((r >> 2) & 3); }
__device__ __forceinline__ int tile_off(int r, int c) { return kRowBytes * r + 16 * (c ^ row_swz(r)); }

typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s_t lds_v4s_t;

typedef __attribute__((address_space(3))) u32x4 lds_u32x4_t;

// transposed 4 x b16 read at LDS byte offset off
__device__ __forceinline__ uint2 lds_read_tr_at(unsigned off) {
  const v4s_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t*)(uintptr_t)off);
  return __builtin_bit_cast(uint2, r);
}

// Logit MFMAs with the accumulator in VGPRs.  The output accumulators take
// all 256 AGPRs, and the compiler puts every MFMA it emits in one register
// file, so the logits product is issued here instead; the compiler does not
// see it as an MFMA, so its hazards are covered by hand:
//   - a VALU write of an operand needs 2 wait states: each MFMA is preceded
//     by s_nop 1;
//   - back-to-back accumulation into the same registers needs none;
//   - a VALU read of the result needs up to 19 (16-pass XDL): wide_s_done
//     waits 24 and pins the result after that point.
__device__ __forceinline__ void mma32_v0(f32x16& c, const Frag<bf16_t>& a, const Frag<bf16_t>& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(c) : "v"(a.v), "v"(b.v));
}
__device__ __forceinline__ void mma32_v(f32x16& c, const Frag<bf16_t>& a, const Frag<bf16_t>& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a.v), "v"(b.v));
}
__device__ __forceinline__ void wide_s_done(f32x16& c) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(c));
}

struct WideShared {
  __attribute__((aligned(16))) char kbuf[kBufs][kTileBytes];
  const char* row_ptr[kRing][kTile];
  int flag[kWideWaves];
  __attribute__((aligned(16))) float rho[2][kTile];          // row factors (normalisation)
};

// Lane offsets of the LDS read patterns.  Derived from the lane id where
// they are used, so nothing lane-dependent stays in a register across the
// loop.
__device__ __forceinline__ int wide_lane() {
  int lid;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lid));
  return lid;
}
// keys: k-step s reads row l % 32, chunk 2 s + l / 32, at k[s % 4] + 128 (s / 4)
// (slot 2 s ^ (l / 32 ^ g) = 8 (s / 4) + (2 (s % 4) ^ (l / 32 ^ g)))
struct KeyOffs { int k[4]; };
__device__ __forceinline__ KeyOffs key_offs() {
  const int lid = wide_lane();
  const int r = lid & 31, x = (lid >> 5) ^ row_swz(r);
  KeyOffs o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o.k[i] = kRowBytes * r + 16 * ((2 * i) ^ x);
  return o;
}
// values: k-step u, read w (rows 16 u + 8 w + 4 (l / 32) + 0..3) of dim
// block db at v[u][w][db % 2] + 128 (db / 2).  16-lane group G reads dims
// 16 (G % 2) .. + 15 of the block: lane c of the group row c / 4 of a 4-row
// run and the 4 dims 4 (c % 4) .. + 3, i.e. half c % 2 of chunk
// 4 db + y, y = 2 (G % 2) + (c % 4) / 2, in slot 8 (db / 2) + ((4 (db % 2) + y) ^ g).
struct ValOffs { int v[2][2][2]; };
__device__ __forceinline__ ValOffs val_offs() {
  const int lid = wide_lane();
  const int h = lid >> 5, G = lid >> 4, c = lid & 15;
  const int y = 2 * (G & 1) + ((c & 3) >> 1);
  ValOffs o;
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const int rr = 16 * u + 8 * w + 4 * h + (c >> 2);
#pragma unroll
      for (int p = 0; p < 2; ++p)
        o.v[u][w][p] = kRowBytes * rr + 16 * ((4 * p + y) ^ row_swz(rr)) + 8 * (c & 1);
    }
  return o;
}
// acc + the sum of squares of the two bf16 in w.  w is taken by value: a
// bit cast applied directly to an element of a vector register tuple reads
// element 0 whatever the index.
__device__ __forceinline__ float sumsq_bf16x2(uint32_t w, float acc) {
  const hw_bf16x2_t x = __builtin_bit_cast(hw_bf16x2_t, w);
  return __builtin_amdgcn_fdot2_f32_bf16(x, x, acc, false);
}

// x in the lanes of m, y in the others (one v_cndmask on a scalar lane mask)
__device__ __forceinline__ float sel_lanes(float x, float y, uint64_t m) {
  float r;
  asm("v_cndmask_b32 %0, %1, %2, %3" : "=v"(r) : "v"(y), "v"(x), "s"(m));
  return r;
}

// One block's split.  EXACT = false: the main pass; returns true, without
// writing anything, when a logit left its head's reference band.  EXACT =
// true: the split again, first for each head's exact maximum, then
// accumulating against it, one tile at a time.
//
// NORM: queries and compressed entries are normalised to unit root-mean-
// square over their 576 dims ("DeepSeek V4 comprimeix el context", section
// "CSA: buscar primer i atendre despres": normalisation of queries and
// compressed entries stabilises the logits).  A head's factor 1/rms(q)
// joins its softmax scale; a row's factor g = 1/rms(row) (1 for raw window
// rows) multiplies its logit and, since the normalised entry is also the
// value, its weight in the weighted sum, while the normaliser sums the
// weights without it.  Each tile's g are computed from the tile in LDS by
// all four waves (8 lanes a row) one tile ahead and kept in LDS.
template <bool EXACT, bool NORM>
__device__ __forceinline__ bool wide_split(const AttnArgs& a, WideShared& sh) {
  auto& kbuf = sh.kbuf;
  auto& row_ptr = sh.row_ptr;
  auto& flag = sh.flag;
  // uniform scalars the loop uses, pinned to scalar registers
  const float c_log2 = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, a.c)));
  const float ninf = -INFINITY;
  const hw_bf16x2_t ones_bf16x2 = __builtin_bit_cast(hw_bf16x2_t, 0x3f803f80u);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nblk = gridDim.x * gridDim.y * gridDim.z;
  const int lb = xcd_block(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z), nblk);
  const int split = lb % gridDim.x, hg = (lb / gridDim.x) % gridDim.y, b = lb / (gridDim.x * gridDim.y);
  const int hl = lane & 31, lh = lane >> 5;
  const int head = hg * kWideHeads + wave * 32 + hl;
  const bool hok = head < a.H;
  const bf16_t* q = reinterpret_cast<const bf16_t*>(a.q);
  const char* ent = reinterpret_cast<const char*>(a.entries);
  const char* win = reinterpret_cast<const char*>(a.window);
  const char* safe_row = reinterpret_cast<const char*>(q + (int64_t)b * a.H * kE);

  // queries, the B operand of the logits: k-step s, lane l holds head l % 32
  // and dims 16 s + 8 (l / 32) .. + 7.  A head past H reads head 0 and
  // writes nothing.
  //
  // The main pass stages them through tile buffers 1 and 2 (free until the
  // second tile's copy), in two halves of 288 dims: each wave copies its 32
  // heads' half rows (576 bytes each) into its own 18 KB region with whole
  // 1 KB copies, then reads its fragments from there.  A fragment load from
  // global memory touches 32 heads' rows at once, 32 bytes of a 128-byte
  // line each, so four consecutive loads share every line; a whole-line
  // copy asks for each line once.  Region row r holds chunk j of the half
  // row in slot j ^ f(r), f(r) = (r / 4) % 4: the 16 rows a fragment read
  // serves together then cover all 64 banks.
  Frag<bf16_t> qf[kQSteps];
  auto q_row = [&](int r) {                                  // query row of the wave's head r
    const int hd = hg * kWideHeads + wave * 32 + r;
    return reinterpret_cast<const char*>(q + ((int64_t)b * a.H + (hd < a.H ? hd : 0)) * kE);
  };
  const unsigned q_region = lds_offset(kbuf[1]) + 18432 * wave;    // buffers 1 and 2
  auto q_stage = [&](int half) {
#pragma unroll
    for (int n = 0; n < 18; ++n) {
      const int slot = 64 * n + lane, r = slot / 36, jj = slot - 36 * r;
      const char* src = q_row(r) + 576 * half + 16 * (jj ^ ((r >> 2) & 3));
      dma16(src, (unsigned)__builtin_amdgcn_readfirstlane(q_region + 1024 * n));
    }
  };
  auto q_read = [&](int half) {
    const int y = lh ^ ((hl >> 2) & 3);
    const unsigned base = q_region + 576 * hl;
    const unsigned o0 = base + 16 * y, o1 = base + 16 * (2 ^ y);
#pragma unroll
    for (int u = 0; u < 9; ++u) {
      qf[18 * half + 2 * u].v = *reinterpret_cast<const lds_u32x4_t*>((uintptr_t)(o0 + 64 * u));
      qf[18 * half + 2 * u + 1].v = *reinterpret_cast<const lds_u32x4_t*>((uintptr_t)(o1 + 64 * u));
    }
  };
  if constexpr (EXACT) {
    const bf16_t* qp = q + ((int64_t)b * a.H + (hok ? head : 0)) * kE + 8 * lh;
#pragma unroll
    for (int s = 0; s < kQSteps; ++s) frag_load(qf[s], qp + 16 * s);
  } else {
    q_stage(0);
  }
  // the head's softmax scale (log2 units), with its query's factor
  float c_head = c_log2;
  auto q_norm = [&]() {
    if constexpr (NORM) {
      float ss = 0.f;
#pragma unroll
      for (int s = 0; s < kQSteps; ++s)
#pragma unroll
        for (int w = 0; w < 4; ++w) ss = sumsq_bf16x2(qf[s].v[w], ss);
      ss += __shfl_xor(ss, 32, 64);                          // the head's other 288 dims
      c_head = c_log2 * __frsqrt_rn(ss * (1.f / kE) + a.norm_eps);
    }
  };
  if constexpr (EXACT) q_norm();

  f32x16 O[kVBlocks];
#pragma unroll
  for (int db = 0; db < kVBlocks; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) O[db][i] = 0.f;
  float m_ref = -INFINITY, l_run = 0.f;

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
  const int s_end = dense_end(a, b, s_begin, min(a.nslots, s_begin + a.slots_per_split));
  const int ntiles = s_end > s_begin ? (s_end - s_begin + kTile - 1) / kTile : 0;

  // Rows of tile t: every wave works out which rows are present (lane r
  // for row r) and returns that mask, uniform; wave 0 also writes the row
  // addresses into ring slot t % kRing for the copies.  A selected entry
  // comes in as e_sel, loaded a tile ahead by sel_load.
  auto sel_load = [&](int t) {
    int e = -1;
    if (lane < kTile && !a.dense) {
      const int s = s_begin + t * kTile + lane;
      if (s < s_end && s < a.k) e = a.idx[(int64_t)b * a.k + s];
    }
    return e;
  };
  auto resolve = [&](int t, int e_sel) {
    int ok_lane = 0;
    if (lane < kTile) {
      const int s = s_begin + t * kTile + lane;
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
      if (wave == 0) row_ptr[t % kRing][lane] = p;
      ok_lane = ok;
    }
    return (uint32_t)__ballot(lane < kTile && ok_lane);     // bit r: row r present
  };
  // Copy i of this wave for tile t (copy n = wave + 4 i of the tile): this
  // lane fills slot q = 64 n + lane of the row-major image, chunk
  // (q % 72) ^ g of row q / 72.
  auto copy_row = [&](int t, int i) {
    const int q = 64 * (wave + kWideWaves * i) + lane;
    return row_ptr[t % kRing][q / (kE / 8)];
  };
  auto copy_off = [&](int i) {
    const int q = 64 * (wave + kWideWaves * i) + lane;
    const int r = q / (kE / 8), j = q - (kE / 8) * r;
    return 16 * (j ^ row_swz(r));
  };
  auto copy_src = [&](int t, int i) { return copy_row(t, i) + copy_off(i); };
  auto copy_issue = [&](const char* src, int k, int i) {
    const unsigned base = lds_offset(kbuf[k]) + 1024 * (wave + kWideWaves * i);
    dma16(src, (unsigned)__builtin_amdgcn_readfirstlane(base));
  };
  // gather tile t into buffer k at once
  auto issue = [&](int t, int k) {
    const char* src[kCopies];
#pragma unroll
    for (int i = 0; i < kCopies; ++i) src[i] = copy_src(t, i);
#pragma unroll
    for (int i = 0; i < kCopies; ++i) copy_issue(src[i], k, i);
  };

  // logits S^T of one tile; piece(s) is issued after the MFMA of k-step s
  // the lane's K read offsets within a tile, computed once per split
  KeyOffs LK = key_offs();
#pragma unroll
  for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(LK.k[i]));
  auto qk = [&](const char* kb, f32x16& S, auto&& piece) {
    // per-lane read addresses of this buffer, pinned so that every read is
    // one of them plus an immediate offset
    const KeyOffs& L = LK;
    unsigned kp[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kp[i] = lds_offset(kb) + L.k[i];
      asm volatile("" : "+v"(kp[i]));
    }
    Frag<bf16_t> K[kKDepth];
    auto kload = [&](int s) {
      K[s % kKDepth].v = *reinterpret_cast<const lds_u32x4_t*>((uintptr_t)(kp[s & 3] + 128 * (s >> 2)));
    };
#pragma unroll
    for (int s = 0; s < kKDepth - 1; ++s) kload(s);
#pragma unroll
    for (int s = 0; s < kQSteps; ++s) {
      if (s + kKDepth - 1 < kQSteps) kload(s + kKDepth - 1);
      if (s == 0) mma32_v0(S, K[0], qf[0]);
      else mma32_v(S, K[s % kKDepth], qf[s]);
      piece(s);
      __builtin_amdgcn_sched_barrier(0);
    }
    wide_s_done(S);
  };
  // O^T += V^T P^T for one tile.  The lane's V^T read offsets within a tile
  // are the same for every tile: computed once, pinned so that they are not
  // recomputed in the loop (33 fewer VALU instructions per tile).
  ValOffs L0 = val_offs();
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int w = 0; w < 2; ++w)
#pragma unroll
      for (int q = 0; q < 2; ++q) asm volatile("" : "+v"(L0.v[u][w][q]));
  auto pv = [&](const char* vb, const Frag<bf16_t>* P, auto&& piece) {
    const ValOffs& L = L0;
    unsigned vp[2][2][2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int w = 0; w < 2; ++w)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          vp[u][w][q] = lds_offset(vb) + L.v[u][w][q];
          asm volatile("" : "+v"(vp[u][w][q]));
        }
    Frag<bf16_t> V[kVDepth];
    // MFMA j: k-step u = j / 16, dim block db = j % 16
    auto vload = [&](int j) {
      const int u = j >> 4, db = j & 15;
      const uint2 x = lds_read_tr_at(vp[u][0][db & 1] + 128 * (db >> 1));
      const uint2 y = lds_read_tr_at(vp[u][1][db & 1] + 128 * (db >> 1));
      V[j % kVDepth].v = u32x4{x.x, x.y, y.x, y.y};
    };
#pragma unroll
    for (int j = 0; j < kVDepth - 1; ++j) vload(j);
#pragma unroll
    for (int j = 0; j < 2 * kVBlocks; ++j) {
      if (j + kVDepth - 1 < 2 * kVBlocks) vload(j + kVDepth - 1);
      mma32(O[j & 15], V[j % kVDepth], P[j >> 4]);
      piece(j);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Row factors of tile t (NORM) from its image kb in LDS, in 11 pieces:
  // wave w takes rows 8w .. 8w+7, 8 lanes a row, each lane 9 chunks of 8
  // elements (piece p loads chunk p and sums the squares of chunk p-1);
  // piece 10 reduces over the row's lanes and writes g: 1 for window rows
  // and for rows the tile's mask leaves out (whose zero weights must stay 0).
  struct RhoSt { u32x4 x; float ss; unsigned base; };
  auto rho_piece = [&](int p, const char* kb, int t, uint32_t mask, RhoSt& rs, float* dst) {
    const int r = 8 * wave + (lane >> 3);
    if (p == 0) {
      rs.ss = 0.f;
      rs.base = lds_offset(kb) + kRowBytes * r + 16 * ((lane & 7) ^ row_swz(r));
    }
    if (p >= 1 && p <= 9) {
#pragma unroll
      for (int w = 0; w < 4; ++w) rs.ss = sumsq_bf16x2(rs.x[w], rs.ss);
    }
    if (p <= 8) rs.x = *reinterpret_cast<const lds_u32x4_t*>((uintptr_t)(rs.base + 128 * p));
    if (p == 10) {
      float ss = rs.ss;
      ss += __shfl_xor(ss, 1, 64);
      ss += __shfl_xor(ss, 2, 64);
      ss += __shfl_xor(ss, 4, 64);
      const int sl = s_begin + t * kTile + r;
      const bool entry_row = ((mask >> r) & 1u) && (a.dense || sl < a.k);
      if ((lane & 7) == 0) dst[r] = entry_row ? __frsqrt_rn(ss * (1.f / kE) + a.norm_eps) : 1.f;
    }
  };
  auto rho_all = [&](const char* kb, int t, uint32_t mask, float* dst) {
    RhoSt rs;
#pragma unroll
    for (int p = 0; p < 11; ++p) rho_piece(p, kb, t, mask, rs, dst);
  };

  // Softmax of one tile in pieces (piece s runs after logit k-step s of the
  // next tile): masked, scaled logits; the tile maximum of the head; the
  // reference (check: the main pass, which sets references and flags logits
  // past the band); the weights, their sum and their bf16 B operands.
  struct Soft {
    float sv[16];
    float mx, m_use, psum;
    int flagged;
    Frag<bf16_t> P[2];
    float rv[2][4], rr[2];                                   // row factors in use (NORM)
  };
  // mask: the tile's row mask (uniform).  Logits stay unscaled until the
  // exponent: c >= 0, so the head's maximum of c l is c times its maximum of
  // l, and exp2(c l - m) is one FMA and the exponential.  The weights' sum is
  // taken over their bf16 values, the ones the weighted sum uses.
  // rt: the tile's row factors (NORM): register i of a lane belongs to row
  // 8 (i / 4) + 4 (l / 32) + i % 4.
  auto soft_piece = [&](int s, const f32x16& S, uint32_t mask, Soft& st, bool check,
                        const float* rt) {
    if (s < 4) {
      if constexpr (NORM) {
        // factors of register group s, loaded one piece ahead
        auto ld4 = [&](int gidx, float* d) {
          const float4 v = *reinterpret_cast<const float4*>(rt + 8 * gidx + 4 * lh);
          d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
        };
        if (s == 0) ld4(0, st.rv[0]);
        if (s < 3) ld4(s + 1, st.rv[(s + 1) & 1]);
      }
#pragma unroll
      for (int i = 4 * s; i < 4 * s + 4; ++i) {
        // register i holds row 8 (i / 4) + 4 (l / 32) + i % 4: lanes 0..31
        // take bit b of the mask, lanes 32..63 bit b + 4
        const int b = 8 * (i >> 2) + (i & 3);
        const uint64_t lo = (mask >> b) & 1u ? 0xffffffffull : 0ull;
        const uint64_t hi = (mask >> (b + 4)) & 1u ? 0xffffffff00000000ull : 0ull;
        const float l = NORM ? S[i] * st.rv[s & 1][i & 3] : S[i];
        st.sv[i] = sel_lanes(l, ninf, lo | hi);
      }
    } else if (s == 4) {
      float m = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) m = fmaxf(m, st.sv[i]);
      st.mx = m;
    } else if (s == 5) {
      const float m = max_xor32(st.mx);
      st.mx = m == -INFINITY ? m : m * c_head;               // the head's tile maximum of c l
    } else if (s == 6) {
      if (check) {
        const bool first = (m_ref == -INFINITY);
        st.flagged |= (!first && st.mx > m_ref + kRefBand) ? 1 : 0;
        m_ref = first ? st.mx : m_ref;
      }
      st.m_use = (m_ref == -INFINITY) ? 0.f : -m_ref;        // negated reference
      st.psum = 0.f;
    } else if (s >= 7 && s < 23) {
      const int i = s - 7;
      st.sv[i] = __builtin_amdgcn_exp2f(fmaf(st.sv[i], c_head, st.m_use));
      if constexpr (NORM) {
        if (!(i & 1)) {                                      // factors of rows i, i+1
          const float2 v = *reinterpret_cast<const float2*>(rt + 8 * (i >> 2) + 4 * lh + (i & 3));
          st.rr[0] = v.x;
          st.rr[1] = v.y;
        }
      }
      if (i & 1) {
        const int k = i >> 1;                                // pair k: slot pair of P[k / 4]
        if constexpr (NORM) {
          // the weighted sum takes the normalised rows (weight times the
          // row factor); the normaliser sums the weights themselves
          const uint32_t pk = pack_bf16x2(st.sv[i - 1] * st.rr[0], st.sv[i] * st.rr[1]);
          st.P[k >> 2].v[k & 3] = pk;
          st.psum += st.sv[i - 1] + st.sv[i];
        } else {
          const uint32_t pk = pack_bf16x2(st.sv[i - 1], st.sv[i]);
          st.P[k >> 2].v[k & 3] = pk;
          st.psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(hw_bf16x2_t, pk), ones_bf16x2,
                                                    st.psum, false);
        }
      }
    } else if (s == 23) {
      l_run += st.psum;
    }
  };
  auto soft_all = [&](const f32x16& S, uint32_t mask, Soft& st, bool check, const float* rt) {
#pragma unroll
    for (int s = 0; s < 24; ++s) soft_piece(s, S, mask, st, check, rt);
  };
  auto any_flag = [&]() {
    int any = 0;
#pragma unroll
    for (int w = 0; w < kWideWaves; ++w) any |= flag[w];
    return any != 0;
  };

  if constexpr (!EXACT) {
    // prologue: rows of tiles 0..2, selection of tile 3, tile 0 landed and
    // its logits done, tile 1 in flight
    // every ring slot the loop reads holds valid row addresses: slots of
    // tiles past the split resolve to the safe row.  mk[i]: row mask of tile
    // t + i.
    // The selections load while the first query half is in flight; the rows
    // resolve and tile 0 (into buffer 0, which the query does not use) is
    // copied while the second half is.  The selections are settled after the
    // first wait, so that no later use waits for the copies issued since
    // (the compiler does not count them).
    int e0 = sel_load(0), e1 = sel_load(1), e2 = sel_load(2);
    int e_next = sel_load(3);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");        // first query half staged
    asm volatile("" : "+v"(e0), "+v"(e1), "+v"(e2), "+v"(e_next));
    q_read(0);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");      // read before it is overwritten
    q_stage(1);
    uint32_t mk[4];
    mk[0] = resolve(0, e0);
    mk[1] = resolve(1, e1);
    mk[2] = resolve(2, e2);
    __syncthreads();                                         // rows in LDS
    if (ntiles > 0) {
      issue(0, 0);
      asm volatile("s_waitcnt vmcnt(9)" ::: "memory");      // second query half staged (tile 0 may fly)
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    q_read(1);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    q_norm();
    __syncthreads();                                         // query regions free
    f32x16 S;
    if (ntiles > 0) {
      // tiles 0 and 1 in flight together; at most the kCopies copies of
      // tile 1 may still be outstanding once tile 0 has landed
      if (ntiles > 1) {
        issue(1, 1);
        asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      static_assert(kCopies == 9, "the wait above counts one tile's copies");
      __syncthreads();                                       // tile 0 landed
      RhoSt rs0;
      qk(kbuf[0], S, [&](int s) {
        if constexpr (NORM) {
          if (s < 11) rho_piece(s, kbuf[0], 0, mk[0], rs0, sh.rho[0]);
        }
      });
    }
    // A logit past its band sets the wave's flag; the split then runs to the
    // end and the block redoes it (the accumulated values are dropped).
    Soft st;
    st.flagged = 0;
    for (int t = 0; t < ntiles; ++t) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      // the selection loaded last tile is settled here, where nothing is in
      // flight: its use below then waits for no copy of this tile
      asm volatile("" : "+v"(e_next));
      __syncthreads();                                       // tile t+1 landed; tile t-1 fully read
      const uint32_t mt = mk[0];
      if (t + 1 < ntiles) {
        // Between the logit steps: the copies of tile t+2 (row address read
        // two steps ahead; past the last tile the ring holds the safe row,
        // read into the free buffer).  The rows of tile t+3 and the
        // selection of tile t+4 follow between the weighted-sum steps.
        const int kn = (t + 2) % kBufs;
        const char* rp = nullptr;
        // a fresh copy of the logits: the softmax below is then not merged
        // with the last tile's and hoisted ahead of the MFMAs
        uint32_t mtp = mt;
        asm volatile("" : "+v"(S));
        f32x16 Sn;
        qk(kbuf[(t + 1) % kBufs], Sn, [&](int s) {
          soft_piece(s, S, mtp, st, true, sh.rho[t & 1]);
          if ((s & 3) == 0 && (s >> 2) < kCopies) rp = copy_row(t + 2, s >> 2);
          if ((s & 3) == 2 && (s >> 2) < kCopies) copy_issue(rp + copy_off(s >> 2), kn, s >> 2);
        });
        S = Sn;
      } else {
        soft_all(S, mt, st, true, sh.rho[t & 1]);
      }
      // the row factors of tile t+1 (landed at this tile's barrier), read
      // by its softmax in the next tile
      RhoSt rs;
      const bool next_rho = NORM && t + 1 < ntiles;
      pv(kbuf[t % kBufs], st.P, [&](int j) {
        if (j == 8) {
          mk[3] = resolve(t + 3, e_next);
          e_next = sel_load(t + 4);
        }
        if constexpr (NORM) {
          if (next_rho && j >= 12 && j < 23)
            rho_piece(j - 12, kbuf[(t + 1) % kBufs], t + 1, mk[1], rs, sh.rho[(t + 1) & 1]);
        }
      });
      mk[0] = mk[1];
      mk[1] = mk[2];
      mk[2] = mk[3];
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    // the wave's vote is taken with every lane active (inside the lane-0
    // branch it would see lane 0's heads alone)
    const bool wave_flagged = __any(st.flagged);
    if (lane == 0) flag[wave] = wave_flagged;
    __syncthreads();
    const bool redo = ntiles > 0 && any_flag();
    if (redo) return true;
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    auto load_tile = [&](int t) {
      __syncthreads();                                       // buffer and ring free
      const uint32_t m = resolve(t, sel_load(t));
      __syncthreads();
      issue(t, 0);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      return m;
    };
    // the row factors of the loaded tile (NORM), in sh.rho[0]
    auto tile_rho = [&](int t, uint32_t mask) {
      if constexpr (NORM) {
        rho_all(kbuf[0], t, mask, sh.rho[0]);
        __syncthreads();
      }
    };
    float mx = -INFINITY;
    for (int t = 0; t < ntiles; ++t) {
      const uint32_t mt = load_tile(t);
      tile_rho(t, mt);
      f32x16 S;
      qk(kbuf[0], S, [](int) {});
      Soft st;
#pragma unroll
      for (int s = 0; s < 6; ++s) soft_piece(s, S, mt, st, false, sh.rho[0]);
      mx = fmaxf(mx, st.mx);
    }
    m_ref = mx;
    for (int t = 0; t < ntiles; ++t) {
      const uint32_t mt = load_tile(t);
      tile_rho(t, mt);
      f32x16 S;
      qk(kbuf[0], S, [](int) {});
      Soft st;
      st.flagged = 0;
      soft_all(S, mt, st, false, sh.rho[0]);
      pv(kbuf[0], st.P, [](int) {});
    }
  }

  const float LN2 = 0.6931471805599453f;
  const float l = sum_xor32(l_run);
  // the sink joins where the splits end: here with one split, else in the
  // merge
  const float s2 = (a.sink && a.nsplit == 1) ? a.sink[hok ? head : 0] * 1.4426950408889634f
                                             : -INFINITY;
  float inv, lse2;
  head_norm(l, m_ref, s2, &inv, &lse2);
  // Output rows (the result, or with several splits this split's
  // normalised partial, kept in bf16, the output's precision).  Lane l holds
  // head l % 32, dims 32 db + 8 q + 4 (l / 32) + 0..3 in registers 4 q ..
  // 4 q + 3 of block db, so stores straight from the registers would write 8
  // scattered bytes a lane; instead each wave stages its 32 heads through
  // LDS (the tile buffers, free once every wave is past its last tile), 256
  // dims at a time, with 16-byte chunk c of row r at chunk c ^ r, and stores
  // whole 512-byte row segments.
  const bool part = a.nsplit > 1;
  bf16_t* orow0 = part ? reinterpret_cast<bf16_t*>(a.o_part) : reinterpret_cast<bf16_t*>(a.out);
  char* stage = sh.kbuf[0] + 16384 * wave;
  __syncthreads();
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
    for (int d8 = 0; d8 < 8; ++d8)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const f32x16& o = O[8 * hh + d8];
        const uint2 w = make_uint2(pack_bf16x2(o[4 * qq] * inv, o[4 * qq + 1] * inv),
                                   pack_bf16x2(o[4 * qq + 2] * inv, o[4 * qq + 3] * inv));
        *reinterpret_cast<uint2*>(stage + 512 * hl + 16 * ((4 * d8 + qq) ^ hl) + 8 * lh) = w;
      }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 2 * i + lh;                               // row (head) r, chunk hl
      const u32x4 v = *reinterpret_cast<const u32x4*>(stage + 512 * r + 16 * (hl ^ r));
      const int hd = hg * kWideHeads + wave * 32 + r;
      if (hd < a.H) {
        const int64_t row = part ? ((int64_t)b * a.H + hd) * a.nsplit + split : (int64_t)b * a.H + hd;
        *reinterpret_cast<u32x4*>(orow0 + row * kDv + 256 * hh + 8 * hl) = v;
      }
    }
  }
  if (hok && lh == 0) {
    if (part) a.lse_part[((int64_t)b * a.H + head) * a.nsplit + split] = lse2 * LN2;
    else if (a.lse) a.lse[(int64_t)b * a.H + head] = lse2 * LN2;
  }
  return false;
}

template <bool NORM>
__device__ __noinline__ void wide_split_exact(const AttnArgs& a, WideShared& sh) {
  wide_split<true, NORM>(a, sh);
}

template <bool NORM>
__global__ __launch_bounds__(64 * kWideWaves) void attend_wide_kernel(AttnArgs a) {
  __shared__ WideShared sh;
  __shared__ AttnArgs args;
  if (wide_split<false, NORM>(a, sh)) {                      // rare
    // the arguments reach the out-of-line pass through LDS, so that the
    // main pass never needs an addressable copy of them
    if (threadIdx.x == 0) args = a;
    __syncthreads();
    wide_split_exact<NORM>(args, sh);
  }
}

// One wave per (query, head): lse = ln(sum_s exp(lse_s) + exp(sink_h));
// out = sum_s exp(lse_s - lse) o_s (the partials carry no sink; sink may be
// NULL).  Lane l takes the lse of splits l, l + 64, ...; the partial rows
// are loaded eight splits at a time and accumulated in split order, so the
// result does not depend on timing.  P: the partials' type (fp32, or bf16
// for the bf16 attention's own splits).
template <class T, class P>
__global__ __launch_bounds__(256) void merge_kernel(const P* __restrict__ o_part,
                                                    const float* __restrict__ lse_part, int64_t BH,
                                                    int S, const float* __restrict__ sink, int H,
                                                    T* __restrict__ out,
                                                    float* __restrict__ lse) {
  const int lane = threadIdx.x & 63;
  const int64_t bh = (int64_t)xcd_block(blockIdx.x, gridDim.x) * 4 + (threadIdx.x >> 6);
  if (bh >= BH) return;
  const float* lp = lse_part + bh * S;
  if (S <= 8) {
    // up to eight splits: the partial rows are loaded together with the lse
    // values rather than after them (one memory latency, not two).  When
    // every split is empty all weights are 0 and the rows (zeros) add 0.
    float v[8][8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (u < S) {
        Row8<P>::load(o_part + (bh * S + u) * kDv + lane * 8, v[u]);
      } else {
#pragma unroll
        for (int d = 0; d < 8; ++d) v[u][d] = 0.f;
      }
    }
    const float ls = lane < S ? lp[lane] : -INFINITY;
    float m8 = ls;
#pragma unroll
    for (int off = 4; off >= 1; off >>= 1) m8 = fmaxf(m8, __shfl_xor(m8, off, 64));
    m8 = __shfl(m8, 0, 64);                                  // lanes 0..7 hold the splits
    const float sk = sink ? sink[bh % H] : -INFINITY;
    m8 = fmaxf(m8, sk);
    const bool any = m8 != -INFINITY;
    const float wl = (any && lane < S) ? __expf(ls - m8) : 0.f;
    float t8 = wl;
#pragma unroll
    for (int off = 4; off >= 1; off >>= 1) t8 += __shfl_xor(t8, off, 64);
    t8 = __shfl(t8, 0, 64);
    if (any && sk != -INFINITY) t8 += __expf(sk - m8);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float w = __shfl(wl, u, 64);
#pragma unroll
      for (int d = 0; d < 8; ++d) acc[d] = fmaf(w, v[u][d], acc[d]);
    }
    const float inv = t8 > 0.f ? 1.f / t8 : 0.f;
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[d] *= inv;
    Row8<T>::store(out + bh * kDv + lane * 8, acc);
    if (lse && lane == 0) lse[bh] = t8 > 0.f ? m8 + __logf(t8) : -INFINITY;
    return;
  }
  float mx = -INFINITY;
  for (int s = lane; s < S; s += 64) mx = fmaxf(mx, lp[s]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  const float sk = sink ? sink[bh % H] : -INFINITY;
  mx = fmaxf(mx, sk);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float tot = 0.f;
  if (mx != -INFINITY) {
    for (int s0 = 0; s0 < S; s0 += 64) {
      const int n = min(64, S - s0);
      const float wl = lane < n ? __expf(lp[s0 + lane] - mx) : 0.f;   // weight of split s0 + lane
      tot += wl;
      for (int j = 0; j < n; j += 8) {
        float v[8][8];
        float w[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          w[u] = __shfl(wl, j + u, 64);
          if (j + u < n) {
            Row8<P>::load(o_part + (bh * S + s0 + j + u) * kDv + lane * 8, v[u]);
          } else {
#pragma unroll
            for (int d = 0; d < 8; ++d) v[u][d] = 0.f;
          }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
          for (int d = 0; d < 8; ++d) acc[d] = fmaf(w[u], v[u][d], acc[d]);
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) tot += __shfl_xor(tot, off, 64);
    if (sk != -INFINITY) tot += __expf(sk - mx);
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
  // (fp32: one wave a block, so a tile a split when blocks are few)
  const int64_t cap = dt == 0 ? tiles : (tiles / 2 > 1 ? tiles / 2 : 1);
  if (s > cap) s = cap;
  if (s > 64) s = 64;
  if (s < 1) s = 1;
  // bf16 with a full round of blocks: fewer splits can be cheaper.  Each
  // split adds a partial output (written, then read by the merge) that costs
  // about 1.1 tiles of the wide kernel, so take the split count in
  // [s/2, s] with the least tiles-per-split + 1.1 * splits (measured: 36
  // tiles over 32 queries run in 45.5 us as 6 splits of 6 tiles against
  // 48.5 us as 8 splits of up to 5; 256 tiles keep 8 splits).
  if (dt == 1 && blocks * s >= 256 && s > 1) {
    int64_t best = s, best_cost = -1;
    for (int64_t c = (s + 1) / 2; c <= s; ++c) {
      const int64_t per_c = (tiles + c - 1) / c;
      const int64_t cost = 10 * per_c + 11 * c;
      if (best_cost < 0 || cost < best_cost) { best = c; best_cost = cost; }
    }
    s = best;
  }
  // equal whole tiles per split; drop splits that would be empty
  const int64_t per = (tiles + s - 1) / s;
  return (int)((tiles + per - 1) / per);
}

// partial outputs (fp32; bf16 for bf16 calls) and their lse (fp32)
size_t attend_partial_bytes(int dt, int64_t B, int H, int64_t nslots) {
  const int S = attend_splits(dt, B, H, nslots);
  if (S <= 1) return 0;
  return (size_t)B * H * S * (kDv * (dt == 0 ? 4 : 2) + 4) + 256;
}

template <class T>
static hipError_t launch_attend_t(const AttendParams& p, void* ws, hipStream_t stream) {
  typedef AttnCfg<T> C;
  (void)sizeof(C);
  AttnArgs a;
  a.q = p.q; a.entries = p.entries; a.window = p.window; a.idx = p.idx; a.q_pos = p.q_pos;
  a.ent_bstride = p.ent_bstride; a.win_bstride = p.win_bstride; a.win_pos0 = p.win_pos0;
  a.win_rows = p.win_rows; a.dense = p.dense; a.hm = p.hm; a.sink = p.sink;
  a.N = p.N; a.B = (int)p.B; a.H = p.H; a.W = p.dense ? 0 : p.W; a.k = p.dense ? 0 : p.k;
  a.nslots = (int)(p.dense ? p.N : (int64_t)p.k + p.W);
  // scale >= 0 (checked by the caller).  Scale 0 (uniform weights) runs as
  // the smallest normal scale: the logits are then indistinguishable from 0,
  // and a missing row (logit -inf) still gets weight 0 rather than NaN.
  a.c = p.scale > 0.f ? p.scale * 1.4426950408889634f : 1.17549435e-38f;
  a.out = p.out; a.lse = p.lse;
  const int S = attend_splits(p.dt, p.B, p.H, a.nslots);
  const int64_t tiles = (a.nslots + kTile - 1) / kTile;
  a.nsplit = S;
  a.slots_per_split = (int)(((tiles + S - 1) / S) * kTile);
  a.o_part = (float*)ws;                                     // bf16 partials for bf16 calls
  a.lse_part = (float*)((char*)ws + (size_t)p.B * p.H * S * kDv * sizeof(T));
  const int hpb = attend_heads_per_block(p.dt, p.H);
  dim3 grid(S, (p.H + hpb - 1) / hpb, (unsigned)p.B);
  const bool norm = p.norm_eps >= 0.f;
  a.norm_eps = norm ? p.norm_eps : 0.f;
  if constexpr (sizeof(T) == 2) {
    if (norm) hipLaunchKernelGGL(attend_wide_kernel<true>, grid, dim3(64 * kWideWaves), 0, stream, a);
    else hipLaunchKernelGGL(attend_wide_kernel<false>, grid, dim3(64 * kWideWaves), 0, stream, a);
  } else {
    if (norm) hipLaunchKernelGGL((attend_kernel<T, 1, true>), grid, dim3(64 * C::NW), 0, stream, a);
    else hipLaunchKernelGGL((attend_kernel<T, 1, false>), grid, dim3(64 * C::NW), 0, stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S == 1) return e;
  const int64_t BH = p.B * p.H;
  hipLaunchKernelGGL((merge_kernel<T, T>), dim3((unsigned)((BH + 3) / 4)), dim3(256), 0, stream,
                     reinterpret_cast<const T*>(a.o_part), a.lse_part, BH, S, p.sink, p.H, (T*)p.out, p.lse);
  return hipGetLastError();
}

// MX entry rows -> bf16 rows for the attention kernels, one 8-element
// chunk (its codes and its block's scale) per thread, 72 per row.  BITS = 4:
// MXFP4 (a 32-bit code word, E2M1 elements); BITS = 8: MXFP8 with E4M3
// elements (two 32-bit code words).  The scaled conversions of gfx950 give
// the exact products while they are bf16 normals.
// Dense (idx == NULL): output row r = b * N + i is entry i of sequence b
// (ent_bstride rows apart; one sequence when it is 0).  Gathered: output row
// r = b * k + j is entry idx[b][j] of sequence b, and idx_out[r] = j, or -1
// with a zero row where the selection holds no entry.
template <int BITS>
__global__ __launch_bounds__(256) void mx_rows_kernel(const uint8_t* codes, const uint8_t* scales,
                                                      const int32_t* idx, int64_t rows, int k,
                                                      int64_t N, int64_t ent_bstride,
                                                      bf16_t* out, int32_t* idx_out) {
  constexpr int kChunks = kE / 8;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= rows * kChunks) return;
  const int64_t r = t / kChunks;
  const int c = (int)(t - r * kChunks);
  int64_t src = -1;
  if (!idx) {
    src = (r / N) * ent_bstride + r % N;
  } else {
    const int64_t b = r / k;
    const int e = idx[r];
    if (e >= 0 && e < N) src = b * ent_bstride + e;
    if (c == 0) idx_out[r] = src >= 0 ? (int32_t)(r - b * k) : -1;
  }
  u32x4 v = u32x4{0u, 0u, 0u, 0u};
  if (src >= 0) {
    const float sc = __uint_as_float(e8m0_f32_bits(scales[src * (kE / 32) + c / 4]));
    if constexpr (BITS == 4) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(codes + src * (kE / 2) + 4 * c);
      v = fp4x8_to_bf16(w, sc);
    } else {
      const uint2 w = *reinterpret_cast<const uint2*>(codes + src * kE + 8 * c);
      v = fp8x8_to_bf16(w.x, w.y, sc);
    }
  }
  *reinterpret_cast<u32x4*>(out + r * kE + 8 * c) = v;
}

hipError_t launch_mx_rows(int bits, const uint8_t* codes, const uint8_t* scales, const int32_t* idx,
                          int64_t rows, int k, int64_t N, int64_t ent_bstride, void* out,
                          int32_t* idx_out, hipStream_t stream) {
  const int64_t threads = rows * (kE / 8);
  if (threads == 0) return hipSuccess;
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (bits == 8)
    hipLaunchKernelGGL(mx_rows_kernel<8>, grid, dim3(256), 0, stream, codes, scales, idx, rows, k,
                       N, ent_bstride, (bf16_t*)out, idx_out);
  else
    hipLaunchKernelGGL(mx_rows_kernel<4>, grid, dim3(256), 0, stream, codes, scales, idx, rows, k,
                       N, ent_bstride, (bf16_t*)out, idx_out);
  return hipGetLastError();
}

hipError_t launch_attend(const AttendParams& p, void* ws, hipStream_t stream) {
  if (p.dt == 0) return launch_attend_t<float>(p, ws, stream);
  return launch_attend_t<bf16_t>(p, ws, stream);
}

hipError_t launch_merge(int dt, const float* o_part, const float* lse_part, int64_t BH, int S,
                        const float* sink, int H, void* out, float* lse, hipStream_t stream) {
  if (dt == 0)
    hipLaunchKernelGGL((merge_kernel<float, float>), dim3((unsigned)((BH + 3) / 4)), dim3(256), 0, stream,
                       o_part, lse_part, BH, S, sink, H, (float*)out, lse);
  else
    hipLaunchKernelGGL((merge_kernel<bf16_t, float>), dim3((unsigned)((BH + 3) / 4)), dim3(256), 0, stream,
                       o_part, lse_part, BH, S, sink, H, (bf16_t*)out, lse);
  return hipGetLastError();
}

}  // namespace cskv
