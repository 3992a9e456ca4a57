/*
 * CPU oracle for token-axis compressed attention (CSA / HCA).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * definition of what the GPU hot path computes.  Only the tests, the smoke
 * check and the CPU-baseline leg of the benchmark load it.  The GPU library
 * never links, includes or calls it, and it shares no code with the GPU
 * library: it decodes the stored input bytes itself and computes everything
 * in fp64 with plain loops.  OpenMP splits only independent outputs, so the
 * result does not depend on the thread count.
 *
 * Sources (the web pages describing the method):
 *  [P1] "Frontier Techniques: NTK RoPE, CSA+HCA, QAT, MTP", section 2.1
 *       "CSA - compress AND select" and 2.2 "HCA - compress harder, attend
 *       everywhere".
 *  [P2] "The State and Signal Problem: MLA and Multi-Token Prediction",
 *       section "MLA compresses what generation must remember" (512-dim
 *       shared latent plus a 64-dim decoupled RoPE key).
 *  [P4] "DeepSeek V4 comprimeix el context: aixi funcionen CSA i HCA",
 *       sections "DeepSeek comprimeix la dimensio temporal" (512-dim shared
 *       KV, content-dependent per-dimension softmax weights), "Finestres
 *       solapades per evitar fronteres artificials" (overlapping windows,
 *       incomplete block stays raw), "CSA: buscar primer i atendre despres"
 *       (indexer, top entries, attention over chosen entries plus the local
 *       window) and "HCA: un resum global 128 vegades mes curt" (dense
 *       attention over all heavily compressed entries).
 *
 * Readings where the pages leave a detail open (each is listed with its
 * reason in the design notes of the repository):
 *  - window of entry i = tokens [(i-1)m, (i+1)m): 2m tokens, stride m;
 *    entry count N = floor(T/m); tokens past N*m stay raw;
 *  - tokens before 0 are absent from the softmax (not zero-padded);
 *  - bias b[p][d] is indexed by position p in the window (p = 0 oldest);
 *  - compressor softmax has no temperature: softmax_p(z + b);
 *  - indexer score = scale * dot(qI, kI) over 64 dims; causal visibility of
 *    entry i for a query at position pos: (i+1)m <= pos+1;
 *  - top-k order: score descending, then index ascending; -1 padding;
 *  - CSA attention: one joint softmax over selected entries and window rows;
 *    logits use all 576 dims, values are dims 0..511;
 *  - attention-sink logits: one more softmax term per head with a zero value;
 *  - query / compressed-entry normalisation (optional): unit root-mean-square
 *    over all 576 dims with an epsilon argument, no learned gain; the
 *    normalised entry is key and value; raw window rows are not normalised;
 *  - MXFP4 (named by [P1] for the indexer's QK path and, as FP4 with block
 *    scales, by "Compressed attention - CSA / HCA" section 3 for the V4.1 KV
 *    cache): the OCP Microscaling v1.0 format, element 2j in the low nibble
 *    of byte j, one E8M0 scale per 32 elements in a separate array;
 *  - FP8 entry rows with block scales: the OCP MXFP8 format with E4M3
 *    elements, one byte an element, one E8M0 scale per 32 elements.
 *
 * All functions return 0 on success and a negative value on bad arguments.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1
#define ORC_E4M3 2
#define ORC_F64 3   /* values already decoded (MXFP4 rows, see below) */

/* ---- decoding of stored inputs (fp32, bf16, OCP fp8 e4m3fn) ------------- */

/* OCP 8-bit floating point, E4M3 variant: 1 sign bit, 4 exponent bits with
 * bias 7, 3 mantissa bits, no infinities, S.1111.111 is NaN, largest finite
 * value 448, subnormals m * 2^-9. */
double cskv_oracle_e4m3_value(uint8_t code) {
  int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(1.0 + m / 8.0, e - 7);
  return s ? -v : v;
}

/* bf16 is the upper half of an IEEE binary32. */
double cskv_oracle_bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* ---- MXFP4 [P1 "QAT": the indexer's QK path runs in FP4 (MXFP4)].  The
 * pages name the format only; its definition is the OCP Microscaling
 * Formats (MX) specification v1.0: a block of 32 FP4 E2M1 elements shares
 * one E8M0 scale, and element i of a block is worth scale * P_i.
 *
 * E2M1: 1 sign bit, 2 exponent bits with bias 1, 1 mantissa bit, no
 * infinities or NaN; exponent 0 is subnormal (m * 0.5); largest value 6. */
double cskv_oracle_e2m1_value(uint8_t code) {
  int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  double v = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -v : v;
}

/* E8M0: an unsigned biased exponent X (bias 127) and no mantissa: 2^(X-127);
 * X = 255 is NaN. */
double cskv_oracle_e8m0_value(uint8_t x) { return x == 255 ? NAN : ldexp(1.0, (int)x - 127); }

/* Rows of `cols` elements (a multiple of 32) in cols/32 MX blocks: codes
 * [rows][cols/2], element 2j in the low nibble of byte j and element 2j+1 in
 * its high nibble; scales [rows][cols/32], scale b covering elements
 * 32b .. 32b+31.  out [rows][cols]. */
int cskv_oracle_mxfp4_decode(const uint8_t* codes, const uint8_t* scales, int64_t rows, int cols,
                             double* out) {
  if (!codes || !scales || !out || rows < 0 || cols <= 0 || cols % 32) return -1;
  for (int64_t r = 0; r < rows; ++r)
    for (int i = 0; i < cols; ++i) {
      const uint8_t byte = codes[r * (cols / 2) + i / 2];
      const uint8_t code = (i & 1) ? (byte >> 4) : (byte & 15);
      out[r * cols + i] =
          cskv_oracle_e8m0_value(scales[r * (cols / 32) + i / 32]) * cskv_oracle_e2m1_value(code);
    }
  return 0;
}

/* ---- MXFP8 entry rows ("Compressed attention - CSA / HCA", section 3: the
 * compressed KV cache is kept in low-bit floating point with block scales).
 * FP8 with block scales is read as the OCP Microscaling v1.0 MXFP8 format
 * with E4M3 elements: a block of 32 E4M3 elements shares one E8M0 scale,
 * and element i of a block is worth scale * E4M3 value.  Codes [rows][cols]
 * (one byte an element), scales [rows][cols/32].  out [rows][cols]. */
int cskv_oracle_mxfp8_decode(const uint8_t* codes, const uint8_t* scales, int64_t rows, int cols,
                             double* out) {
  if (!codes || !scales || !out || rows < 0 || cols <= 0 || cols % 32) return -1;
  for (int64_t r = 0; r < rows; ++r)
    for (int i = 0; i < cols; ++i)
      out[r * cols + i] = cskv_oracle_e8m0_value(scales[r * (cols / 32) + i / 32]) *
                          cskv_oracle_e4m3_value(codes[r * cols + i]);
  return 0;
}

static double ld(const void* buf, int64_t i, int dt) {
  switch (dt) {
    case ORC_F32: return (double)((const float*)buf)[i];
    case ORC_BF16: return cskv_oracle_bf16_value(((const uint16_t*)buf)[i]);
    case ORC_F64: return ((const double*)buf)[i];
    default: return cskv_oracle_e4m3_value(((const uint8_t*)buf)[i]);
  }
}

static int dt_ok(int dt) { return dt == ORC_F32 || dt == ORC_BF16 || dt == ORC_E4M3 || dt == ORC_F64; }

/* ---- compression [P4 "DeepSeek comprimeix la dimensio temporal",
 *      "Finestres solapades ..."; P1 2.1 and 2.2] ------------------------- */

int64_t cskv_oracle_num_entries(int64_t T, int m) { return (m > 0 && T >= 0) ? T / m : -1; }

/* For each requested entry i and each dimension d: the window holds tokens
 * j = (i-1)m + p, p = 0..2m-1, those with j >= 0 being present.  Each
 * present token gets logit l_p = z[j][d] + b[p][d]; the weights are the
 * softmax of the logits over the present tokens, taken separately for every
 * dimension d; the entry value is the weighted sum of x[j][d].
 * out is [n_ids][D]. */
int cskv_oracle_compress(const void* x, const void* z, int dt, const float* bias,
                         int64_t T, int64_t D, int m, const int64_t* entry_ids,
                         int64_t n_ids, double* out) {
  if (!x || !z || !bias || !out || D <= 0 || m <= 0 || T < 0 || n_ids < 0 || !dt_ok(dt))
    return -1;
  int64_t N = T / m;
  for (int64_t t = 0; t < n_ids; ++t)
    if (entry_ids[t] < 0 || entry_ids[t] >= N) return -2;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t t = 0; t < n_ids; ++t) {
    int64_t i = entry_ids[t];
    double* logit = (double*)malloc(sizeof(double) * 2 * m);
    for (int64_t d = 0; d < D; ++d) {
      double mx = -INFINITY;
      for (int p = 0; p < 2 * m; ++p) {
        int64_t j = (i - 1) * m + p;
        if (j < 0) continue;
        logit[p] = ld(z, j * D + d, dt) + (double)bias[(int64_t)p * D + d];
        if (logit[p] > mx) mx = logit[p];
      }
      double den = 0.0, num = 0.0;
      for (int p = 0; p < 2 * m; ++p) {
        int64_t j = (i - 1) * m + p;
        if (j < 0) continue;
        double w = exp(logit[p] - mx);
        den += w;
        num += w * ld(x, j * D + d, dt);
      }
      out[t * D + d] = num / den;
    }
    free(logit);
  }
  return 0;
}

/* ---- indexer scores [P1 2.1 "scored cheaply by the Lightning Indexer";
 *      P4 "CSA: buscar primer i atendre despres"] -------------------------- */

/* s[b][i] = scale * sum_r qI[b][r] * kI[i][r]; visible[b][i] = 1 for every
 * entry at decode (q_pos == NULL), else 1 iff (i+1)*m <= q_pos[b] + 1.
 * key_bstride (elements) offsets kI per query (0: one shared key set). */
int cskv_oracle_index_scores(const void* qI, const void* kI, int dt, int64_t B, int64_t N,
                             int64_t I, double scale, int64_t key_bstride,
                             const int64_t* q_pos, int m, double* scores, uint8_t* visible) {
  if (!qI || !kI || !scores || !visible || B < 0 || N < 0 || I <= 0 || !dt_ok(dt)) return -1;
  if (q_pos && m <= 0) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t i = 0; i < N; ++i) {
      double acc = 0.0;
      for (int64_t r = 0; r < I; ++r)
        acc += ld(qI, b * I + r, dt) * ld(kI, b * key_bstride + i * I + r, dt);
      scores[b * N + i] = scale * acc;
      visible[b * N + i] = q_pos ? ((i + 1) * (int64_t)m <= q_pos[b] + 1) : 1;
    }
  }
  return 0;
}

/* ---- top-k [P1 2.1 "attend only top-1024 entries"; P4 "CSA: ..."] ------- */

typedef struct { double s; int64_t i; } scored;

static int by_score_desc_index_asc(const void* pa, const void* pb) {
  const scored* a = (const scored*)pa;
  const scored* b = (const scored*)pb;
  if (a->s > b->s) return -1;
  if (a->s < b->s) return 1;
  return (a->i < b->i) ? -1 : (a->i > b->i);
}

/* idx[b] = the first min(k, visible count) visible entries under the order
 * (score descending, index ascending), then -1 padding. */
int cskv_oracle_topk(const double* scores, const uint8_t* visible, int64_t B, int64_t N, int k,
                     int32_t* idx) {
  if (!scores || !visible || !idx || B < 0 || N < 0 || k <= 0) return -1;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t b = 0; b < B; ++b) {
    scored* v = (scored*)malloc(sizeof(scored) * (N > 0 ? N : 1));
    int64_t n = 0;
    for (int64_t i = 0; i < N; ++i)
      if (visible[b * N + i]) { v[n].s = scores[b * N + i]; v[n].i = i; ++n; }
    qsort(v, (size_t)n, sizeof(scored), by_score_desc_index_asc);
    for (int j = 0; j < k; ++j) idx[b * k + j] = (j < n) ? (int32_t)v[j].i : -1;
    free(v);
  }
  return 0;
}

/* ---- attention [P1 2.1, 2.2; P4 "CSA: ...", "HCA: ..."] ------------------- */

/* Softmax attention of one query head over an explicit list of rows:
 * l_r = scale * sum_{e<E} q[e] * row_r[e]; o[d] = sum_r p_r row_r[d] for
 * d < Dv; lse = ln(sum_r exp(l_r) + exp(sink)).  The attention sink
 * ("DeepSeek V4 comprimeix el context", section "CSA: buscar primer i
 * atendre despres": learned logits that absorb attention mass) is one more
 * softmax term with logit `sink` and a zero value: p_r = exp(l_r) /
 * (sum_r' exp(l_r') + exp(sink)).  sink = -inf: no sink.
 *
 * Normalisation of queries and compressed entries (the same section: the
 * design normalises them to stabilise the logits).  With norm_eps >= 0 the
 * query and every row flagged in is_entry are replaced by x / rms(x), rms(x)
 * = sqrt(sum_e x[e]^2 / E + norm_eps) over all E dims; the normalised entry
 * is both the key and the value.  Rows not flagged (raw window rows) are
 * used as they are.  norm_eps < 0: no normalisation. */
static double inv_rms(const void* buf, int64_t off, int64_t E, int dt, double eps) {
  double ss = 0.0;
  for (int64_t e = 0; e < E; ++e) {
    const double x = ld(buf, off + e, dt);
    ss += x * x;
  }
  return 1.0 / sqrt(ss / (double)E + eps);
}

static void attend_rows(const void* q, int64_t q_off, int dt, const void* const* row_buf,
                        const int64_t* row_off, const unsigned char* is_entry, int64_t n_rows,
                        int64_t E, int64_t Dv, double scale, double sink, double norm_eps,
                        double* out, double* lse) {
  double* l = (double*)malloc(sizeof(double) * (n_rows > 0 ? n_rows : 1));
  double* g = (double*)malloc(sizeof(double) * (n_rows > 0 ? n_rows : 1));   /* row factors */
  const int norm = norm_eps >= 0.0;
  const double gq = norm ? inv_rms(q, q_off, E, dt, norm_eps) : 1.0;
  double mx = sink;
  for (int64_t r = 0; r < n_rows; ++r) {
    g[r] = (norm && is_entry[r]) ? inv_rms(row_buf[r], row_off[r], E, dt, norm_eps) : 1.0;
    double acc = 0.0;
    for (int64_t e = 0; e < E; ++e)
      acc += (gq * ld(q, q_off + e, dt)) * (g[r] * ld(row_buf[r], row_off[r] + e, dt));
    l[r] = scale * acc;
    if (l[r] > mx) mx = l[r];
  }
  if (mx == -INFINITY) {                       /* no rows and no sink */
    for (int64_t d = 0; d < Dv; ++d) out[d] = 0.0;
    *lse = -INFINITY;
    free(l);
    free(g);
    return;
  }
  double den = sink == -INFINITY ? 0.0 : exp(sink - mx);
  for (int64_t r = 0; r < n_rows; ++r) { l[r] = exp(l[r] - mx); den += l[r]; }
  for (int64_t d = 0; d < Dv; ++d) {
    double acc = 0.0;
    for (int64_t r = 0; r < n_rows; ++r) acc += l[r] * (g[r] * ld(row_buf[r], row_off[r] + d, dt));
    out[d] = acc / den;
  }
  *lse = mx + log(den);
  free(l);
  free(g);
}

/* CSA: rows of query b = entries[idx[b][j]] for idx >= 0 (in list order),
 * followed by the window rows.  Decode (q_pos == NULL): the window is rows
 * 0..W-1 of the window buffer.  Prefill: the raw rows at positions
 * max(0, pos-W+1) .. pos, where buffer row 0 holds position win_pos0.
 * Strides (elements) select per-query entries / window (0: shared).
 * q [B][H][E], out [B][H][Dv], lse [B][H]. */
int cskv_oracle_csa_attend(const void* q, const void* entries, const void* window, int dt,
                           int64_t B, int64_t H, int64_t E, int64_t Dv, int64_t N, int64_t W,
                           const int32_t* idx, int64_t k, int64_t ent_bstride,
                           int64_t win_bstride, int64_t win_rows, const int64_t* q_pos,
                           int64_t win_pos0, double scale, const double* sink, double norm_eps,
                           double* out, double* lse) {
  if (!q || !entries || !idx || !out || !lse || B < 0 || H <= 0 || E <= 0 || Dv <= 0 ||
      Dv > E || N < 0 || W < 0 || k <= 0 || !dt_ok(dt))
    return -1;
  if (W > 0 && !window) return -1;
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t j = 0; j < k; ++j)
      if (idx[b * k + j] >= N) return -2;
    if (q_pos && W > 0) {
      int64_t lo = q_pos[b] - W + 1;
      if (lo < 0) lo = 0;
      if (lo - win_pos0 < 0 || q_pos[b] - win_pos0 >= win_rows) return -3;
    }
  }
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t h = 0; h < H; ++h) {
      int64_t cap = k + W;
      const void** buf = (const void**)malloc(sizeof(void*) * cap);
      int64_t* off = (int64_t*)malloc(sizeof(int64_t) * cap);
      unsigned char* ent = (unsigned char*)malloc(cap);
      int64_t n = 0;
      for (int64_t j = 0; j < k; ++j) {
        int32_t i = idx[b * k + j];
        if (i < 0) continue;
        buf[n] = entries;
        off[n] = b * ent_bstride + (int64_t)i * E;
        ent[n] = 1;
        ++n;
      }
      if (W > 0) {
        int64_t lo, hi;
        if (q_pos) {
          hi = q_pos[b];
          lo = hi - W + 1 < 0 ? 0 : hi - W + 1;
          lo -= win_pos0;
          hi -= win_pos0;
        } else {
          lo = 0;
          hi = W - 1;
        }
        for (int64_t r = lo; r <= hi; ++r) {
          buf[n] = window;
          off[n] = b * win_bstride + r * E;
          ent[n] = 0;
          ++n;
        }
      }
      attend_rows(q, (b * H + h) * E, dt, buf, off, ent, n, E, Dv, scale,
                  sink ? sink[h] : -INFINITY, norm_eps, out + (b * H + h) * Dv, lse + b * H + h);
      free(buf);
      free(off);
      free(ent);
    }
  }
  return 0;
}

/* HCA: every query attends densely over the entries it can see; no window.
 * Decode (q_pos == NULL): all N entries.  Prefill chunk: the query at
 * position q_pos[b] sees entry i iff (i+1)*m <= q_pos[b] + 1, the same
 * causal rule as the indexer's (an entry exists once its block of m tokens
 * is complete), i.e. entries 0 .. min(N, (q_pos[b]+1)/m) - 1. */
int cskv_oracle_hca_attend(const void* q, const void* entries, int dt, int64_t B, int64_t H,
                           int64_t E, int64_t Dv, int64_t N, int64_t ent_bstride,
                           const int64_t* q_pos, int m, double scale, const double* sink,
                           double norm_eps, double* out, double* lse) {
  if (!q || !entries || !out || !lse || B < 0 || H <= 0 || E <= 0 || Dv <= 0 || Dv > E ||
      N < 0 || !dt_ok(dt))
    return -1;
  if (q_pos && m <= 0) return -1;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t h = 0; h < H; ++h) {
      int64_t n = N;
      if (q_pos) {
        const int64_t vis = q_pos[b] + 1 < 0 ? 0 : (q_pos[b] + 1) / m;
        n = vis < N ? vis : N;
      }
      const void** buf = (const void**)malloc(sizeof(void*) * (n > 0 ? n : 1));
      int64_t* off = (int64_t*)malloc(sizeof(int64_t) * (n > 0 ? n : 1));
      unsigned char* ent = (unsigned char*)malloc(n > 0 ? n : 1);
      for (int64_t i = 0; i < n; ++i) {
        buf[i] = entries;
        off[i] = b * ent_bstride + i * E;
        ent[i] = 1;
      }
      attend_rows(q, (b * H + h) * E, dt, buf, off, ent, n, E, Dv, scale,
                  sink ? sink[h] : -INFINITY, norm_eps, out + (b * H + h) * Dv, lse + b * H + h);
      free(buf);
      free(off);
      free(ent);
    }
  }
  return 0;
}

/* Thread count of the OpenMP loops (results do not depend on it). */
void cskv_oracle_set_threads(int n) {
#ifdef _OPENMP
  extern void omp_set_num_threads(int);
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int cskv_oracle_max_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}
