/*
 * cskv: token-axis compressed attention (CSA / HCA) for AMD MI355X (gfx950).
 *
 * The method is described by the pages
 *   "Frontier Techniques: NTK RoPE, CSA+HCA, QAT, MTP" (section 2, CSA + HCA),
 *   "DeepSeek V4 comprimeix el context: aixi funcionen CSA i HCA",
 *   "The State and Signal Problem: MLA and Multi-Token Prediction" (section
 *   "MLA compresses what generation must remember": 512-dim shared latent plus
 *   a decoupled 64-dim RoPE key),
 *   "Compressed attention - CSA / HCA" (sections 1-4: token-axis compression,
 *   recent window plus compressed history, cache budgeting, the FP4 KV cache
 *   with block scales).
 *
 * Data layout (row-major, element counts; D = 512, R = 64, E = D + R = 576):
 *   raw_kv, score_logits [T][512]   raw shared-KV rows and compressor logits
 *   pos_bias             [2m][512]  fp32 per-window-position bias
 *   entries              [N][576]   compressed entries: dims 0..511 content
 *                                    (the attention value), 512..575 RoPE part
 *   idx_keys             [N][64]    indexer keys;   q_idx [B][64] queries
 *   window               [rows][576] raw recent rows (512 content + 64 RoPE)
 *   q                    [B][H][576] attention queries
 *   out                  [B][H][512] attention output;  lse [B][H] fp32
 *   idx_out              [B][k]     int32 selected entries: valid indices in
 *                                    ascending order, then -1 padding
 * MXFP4 storage (the *_mxfp4 calls; OCP Microscaling v1.0, 32 FP4 E2M1
 * elements per E8M0 scale): a row of C elements is C/2 code bytes (element
 * 2j in the low nibble of byte j) plus C/32 scale bytes in a separate array;
 *   entry codes / scales [N][288] / [N][18];  key codes / scales [N][32] / [N][2].
 * MXFP8 storage (the *_mxfp8 calls; 32 FP8 E4M3 elements per E8M0 scale):
 *   entry codes / scales [N][576] / [N][18].
 * Per-query caches: *_bstride gives the element offset between the caches of
 * consecutive queries (0 = one cache shared by all queries).
 *
 * Conventions
 *  - Every pointer argument except `stream` is device memory (or host-pinned
 *    memory the GPU can read), owned by the caller; the library allocates and
 *    frees nothing and keeps no device state between calls (the one
 *    exception is the allocation-free selection call, which uses a fixed
 *    scratch array of the library's on each GPU).  On the host it keeps, per
 *    GPU, the stream its one-launch decode selections run on (see
 *    cskv_index_topk).
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *    stream) and never synchronize the device.
 *  - All arguments are validated before anything is launched: on error
 *    nothing is written and a negative status is returned; the message is
 *    kept per thread in cskv_last_error().
 *  - Inputs outside what the kernels are built for are rejected with
 *    CSKV_ERR_UNSUPPORTED; there is no fallback path.
 *  - Results are deterministic for fixed shapes (fixed split counts and merge
 *    order; the selected set is fully ordered by score then index).
 *  - Tensors must be 16-byte aligned (MXFP4 scale arrays: 1-byte entry
 *    scales, 2-byte aligned key scales).
 */
#ifndef CSKV_H
#define CSKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSKV_VERSION 10500 /* major*10000 + minor*100: 1.5 (query / entry normalisation) */

typedef enum cskv_dtype {
  CSKV_F32 = 0,       /* IEEE binary32 */
  CSKV_BF16 = 1,      /* bfloat16 */
  CSKV_FP8_E4M3 = 2   /* OCP fp8 E4M3 (max 448); indexer keys/queries only */
} cskv_dtype;

typedef enum cskv_status {
  CSKV_OK = 0,
  CSKV_ERR_INVALID_ARG = -1,  /* null pointer, bad size, range out of bounds */
  CSKV_ERR_UNSUPPORTED = -2,  /* valid but outside the compiled kernels */
  CSKV_ERR_WORKSPACE = -3,    /* workspace missing or too small */
  CSKV_ERR_HIP = -4           /* launch failure; HIP message in cskv_last_error() */
} cskv_status;

int cskv_version(void);
const char* cskv_status_string(int status);
/* Message of the last failing call on this thread ("" if none). */
const char* cskv_last_error(void);

/*
 * Compression ("DeepSeek V4 comprimeix el context", sections "DeepSeek
 * comprimeix la dimensio temporal" and "Finestres solapades per evitar
 * fronteres artificials"; "Frontier Techniques", 2.1 m = 4 and 2.2 m' = 128).
 *
 * For entries i in [entry_begin, entry_end) and d < 512:
 *   out[i*ld_out + d] = sum_p w_p[d] * raw_kv[j][d],   j = (i-1)*m + p,
 *   w[d] = softmax over the present p in [0, 2m) (j >= 0) of
 *          score_logits[j][d] + pos_bias[p][d].
 * Entry count N = floor(T/m); tokens past N*m are not compressed (they stay
 * in the raw window).  Only columns 0..511 of each out row are written, so
 * out may be the packed 576-wide entry buffer (ld_out = 576).  Bulk use is
 * (0, N); streaming decode appends one entry per completed block with
 * (N-1, N).
 *   raw_kv, score_logits: [T][512] in dt (F32 or BF16); pos_bias: [2m][512]
 *   fp32; out: rows of ld_out >= 512 elements in dt (ld_out % 8 == 0).
 * An empty entry range is a no-op (the pointers are then not used).
 * Errors: INVALID_ARG for null pointers, T < 0, m < 1, entry range outside
 * [0, N], ld_out < 512; UNSUPPORTED for dt not F32/BF16.
 */
int cskv_compress(const void* raw_kv, const void* score_logits, const float* pos_bias, int64_t T,
                  int32_t m, int64_t entry_begin, int64_t entry_end, void* out, int64_t ld_out,
                  cskv_dtype dt, void* stream);

/*
 * Two-scale compression in one pass over the raw rows (the CSA scale
 * m_small and the HCA scale m_large = R * m_small, "Frontier Techniques" 2.1
 * and 2.2 compress the same history at m = 4 and m' = 128).  Writes exactly
 * what cskv_compress(.., m_small, 0, floor(T/m_small), out_small, ..) and
 * cskv_compress(.., m_large, 0, floor(T/m_large), out_large, ..) write, with
 * one read of raw_kv and score_logits instead of two.
 *   bias_small [2*m_small][512], bias_large [2*m_large][512] fp32;
 *   out_small / out_large rows of ld >= 512 (multiple of 8) in dt.
 *   workspace: cskv_compress2_workspace_size(T, m_large) bytes: the
 *   half-window sums that join the entries at the boundaries between thread
 *   blocks (when the two scales run as separate passes, none is used).
 * bias_large and out_large are not used (may be NULL) when T < m_large.
 * Errors: INVALID_ARG (null pointers, T < 0, m_large not a multiple of
 * m_small, ld < 512); UNSUPPORTED (m_small > 4, m_large > 65536, dt not
 * F32/BF16); WORKSPACE.
 */
size_t cskv_compress2_workspace_size(int64_t T, int32_t m_large);
int cskv_compress2(const void* raw_kv, const void* score_logits, int64_t T,
                   const float* bias_small, int32_t m_small, void* out_small, int64_t ld_small,
                   const float* bias_large, int32_t m_large, void* out_large, int64_t ld_large,
                   cskv_dtype dt, void* workspace, size_t ws_bytes, void* stream);

/*
 * Indexer scoring and top-k selection ("Frontier Techniques", 2.1: entries
 * scored cheaply by the indexer, top-1024 kept; "DeepSeek V4 comprimeix el
 * context", section "CSA: buscar primer i atendre despres").
 *
 *   s[b][i] = idx_scale * sum_{r<64} q_idx[b][r] * idx_keys[b*key_bstride + i*64 + r]
 * Visible entries: all N at decode (q_pos == NULL); for a causal prefill
 * query at position q_pos[b], entry i is visible iff (i+1)*m <= q_pos[b]+1.
 * idx_out[b] receives the min(k, visible) visible entries that come first in
 * the order (score descending, index ascending), as ascending indices,
 * followed by -1 padding.
 *   q_idx [B][64], idx_keys [N][64] (per query if key_bstride > 0), both in
 *   idx_dt (F32, BF16 or FP8_E4M3; for FP8 pass idx_scale = scale_q*scale_k).
 *   workspace: at least cskv_index_topk_workspace_size(B, N, k) bytes.  With
 *     per-query keys (key_bstride > 0), a workspace of at least
 *     cskv_index_topk_per_seq_workspace_size(B, N, k) bytes also keeps the
 *     raw scores between the selection's two passes, so that every key is
 *     read from memory once instead of twice (same result).
 *   Decode selections (q_pos == NULL, shared keys, B <= 32, at least one
 *   compute unit per query, and up to 1,024 keys per compute unit for 17 to
 *   32 queries, 2,048 for 16 or fewer) run as one kernel whose blocks wait
 *   for each other between phases: one block of 1024 threads per compute unit,
 *   every block resident at once (blocks that start late, behind other work
 *   on the GPU, are waited for).  Two such kernels must not run at once, so
 *   they run on one stream per GPU, that of the first such call: once a call
 *   comes on another stream, it and every later decode selection on that
 *   GPU take the multi-launch path, as do calls under stream capture.  Same
 *   result either way; the same workspace.
 * Errors: INVALID_ARG (null pointers, B < 1, N < 1, k < 1, m < 1 with q_pos);
 * UNSUPPORTED (k > 4096); WORKSPACE.
 */
size_t cskv_index_topk_workspace_size(int64_t B, int64_t N, int32_t k);
size_t cskv_index_topk_per_seq_workspace_size(int64_t B, int64_t N, int32_t k);
int cskv_index_topk(const void* q_idx, const void* idx_keys, int64_t B, int64_t N, int32_t k,
                    int64_t key_bstride, const int64_t* q_pos, int32_t m, float idx_scale,
                    cskv_dtype idx_dt, int32_t* idx_out, void* workspace, size_t ws_bytes,
                    void* stream);

/*
 * cskv_index_topk without a workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, serving loops and harnesses
 * that forbid allocation.  The same selection as cskv_index_topk (the same
 * kernels; bit-identical idx_out), with its scratch in a fixed device array
 * of cskv_index_topk_noalloc_max_bytes() bytes (32 MiB) that the library
 * holds on every GPU it runs on until the process ends.  Nothing is
 * allocated or freed by the call.
 *   Selections whose cskv_index_topk_workspace_size(B, N, k) (or, with
 *   per-query keys, less than the per-sequence size: the two-read path)
 *   exceeds that size are rejected with CSKV_ERR_UNSUPPORTED.  Up to 1M
 *   entries at k = 1024 fit for a few dozen queries.
 *   Every call on a GPU uses that GPU's one scratch array: calls that
 *   overlap on one GPU (different streams, or threads) race and must be
 *   serialised by the caller.  Every scratch byte a call reads it first
 *   writes, except the phase words of the one-launch decode selection,
 *   which it compares with 64-bit values unique to the call; nothing
 *   carries over from the previous call.
 * Arguments and the other errors are those of cskv_index_topk.
 */
size_t cskv_index_topk_noalloc_max_bytes(void);
int cskv_index_topk_noalloc(const void* q_idx, const void* idx_keys, int64_t B, int64_t N, int32_t k,
                            int64_t key_bstride, const int64_t* q_pos, int32_t m, float idx_scale,
                            cskv_dtype idx_dt, int32_t* idx_out, void* stream);

/*
 * Indexer scoring and top-k selection over MXFP4 queries and keys ("Frontier
 * Techniques: NTK RoPE, CSA+HCA, QAT, MTP", QAT: the indexer's QK path runs
 * in FP4, MXFP4).  Same selection as cskv_index_topk; only the storage of
 * q_idx and idx_keys differs.  MXFP4 is the OCP Microscaling v1.0 format: a
 * block of 32 FP4 E2M1 elements shares one E8M0 scale 2^(X-127), and each
 * element is worth scale * E2M1 value.
 *   q_codes [B][32] and key_codes [N][32] bytes (per query if key_bstride > 0):
 *     the 64 E2M1 codes of a row, element 2j in the low nibble of byte j and
 *     element 2j+1 in the high nibble.  16-byte aligned.
 *   q_scales [B][2] and key_scales [N][2] bytes: E8M0 scales of elements
 *     0..31 and 32..63 of each row.  2-byte aligned.
 *   key_bstride: rows (not elements) between the key sets of consecutive
 *     queries, 0 for keys shared by all queries.
 *   s[b][i] = idx_scale * sum_r q[b][r] * key[i][r] over the decoded values,
 *   accumulated in fp32; it is exact while every product and partial sum is
 *   an fp32 normal number (as for fp32 inputs).  Scale bytes 0 and 255 decode
 *   to 2^-127 and NaN; rows with NaN scores have no defined rank.
 *   workspace: as cskv_index_topk (per-query keys read once with
 *   cskv_index_topk_per_seq_workspace_size(B, N, k) bytes).
 * Errors: as cskv_index_topk, and INVALID_ARG for null or odd scale pointers.
 */
int cskv_index_topk_mxfp4(const void* q_codes, const uint8_t* q_scales, const void* key_codes,
                          const uint8_t* key_scales, int64_t B, int64_t N, int32_t k,
                          int64_t key_bstride, const int64_t* q_pos, int32_t m, float idx_scale,
                          int32_t* idx_out, void* workspace, size_t ws_bytes, void* stream);

/*
 * Sparse attention over selected entries plus the raw window ("Frontier
 * Techniques", 2.1: attention over the top entries plus a 128-token raw
 * window; "DeepSeek V4 comprimeix el context", section "CSA: ...": full
 * attention over the chosen blocks and the local window).
 *
 * Rows of query b: entries[b*ent_bstride + idx[b][j]*576] for idx[b][j] >= 0,
 * then the window rows: at decode (q_pos == NULL) rows 0..W-1 of
 * window + b*win_bstride; at prefill the raw rows at positions
 * max(0, q_pos[b]-W+1) .. q_pos[b], where row 0 of the window buffer holds
 * position win_pos0 (the buffer has win_rows rows).  For every head h:
 *   l_r = scale * sum_{e<576} q[b][h][e] * row_r[e],
 *   out[b][h][d] = sum_r exp(l_r) * row_r[d] / Z  (d < 512),
 *   lse[b][h] = ln Z,  Z = sum_r exp(l_r) + exp(sink[h])   (lse may be NULL).
 * One softmax covers the selected entries and the window together.
 * sink [H] fp32 (nullable: no sink term) holds per-head attention-sink
 * logits ("DeepSeek V4 comprimeix el context", section "CSA: buscar primer i
 * atendre despres": learned logits that absorb attention mass), in the
 * units of l; a query with no rows then gets out = 0 and lse = sink[h].
 * norm_eps >= 0 normalises the queries and the compressed entries (the same
 * section: their normalisation stabilises the logits): q[b][h] and every
 * selected entry row are divided by sqrt(mean over their 576 dims of x^2 +
 * norm_eps) before the formulas above, so a normalised entry is both the
 * key and the value; raw window rows are used as given.  norm_eps < 0: no
 * normalisation.
 *   idx [B][k] int32 (-1 = no entry; any order); q, entries, window, out in dt
 *   (F32 or BF16); workspace: cskv_attend_workspace_size(...) bytes.
 * scale must be >= 0 and finite (0 gives uniform weights over the rows).
 * Errors: INVALID_ARG (null pointers, sizes < 0, window positions outside the
 * buffer, scale < 0 or not finite, norm_eps NaN or infinite); UNSUPPORTED (dt
 * not F32/BF16); WORKSPACE.
 */
size_t cskv_attend_workspace_size(int64_t B, int32_t H, int64_t rows_per_query);
int cskv_sparse_attend(const void* q, const void* entries, const void* window, const int32_t* idx,
                       int64_t B, int32_t H, int64_t N, int32_t W, int32_t k, int64_t ent_bstride,
                       int64_t win_bstride, int64_t win_rows, const int64_t* q_pos,
                       int64_t win_pos0, float scale, const float* sink, float norm_eps,
                       cskv_dtype dt, void* out, float* lse, void* workspace, size_t ws_bytes,
                       void* stream);

/*
 * CSA: cskv_index_topk followed by cskv_sparse_attend, on one stream, with
 * one workspace of cskv_csa_workspace_size(B, H, N, W, k) bytes.  idx_out
 * ([B][k] int32) receives the selection.
 */
size_t cskv_csa_workspace_size(int64_t B, int32_t H, int64_t N, int32_t W, int32_t k);
int cskv_csa_attend(const void* q, const void* q_idx, const void* entries, const void* idx_keys,
                    const void* window, int64_t B, int32_t H, int64_t N, int32_t W, int32_t k,
                    int32_t m, int64_t ent_bstride, int64_t key_bstride, int64_t win_bstride,
                    int64_t win_rows, const int64_t* q_pos, int64_t win_pos0, float scale,
                    const float* sink, float norm_eps, float idx_scale, cskv_dtype dt,
                    cskv_dtype idx_dt, void* out, float* lse, int32_t* idx_out, void* workspace,
                    size_t ws_bytes, void* stream);

/*
 * HCA ("Frontier Techniques", 2.2; "DeepSeek V4 comprimeix el context",
 * section "HCA: un resum global 128 vegades mes curt"): every query attends
 * densely over the entries it sees, no selection and no window.  Same
 * formulas as cskv_sparse_attend with rows = entries[b*ent_bstride + i*576]:
 *   q_pos == NULL (decode): i < N;
 *   q_pos != NULL (a prefill chunk, positions q_pos[b]): i < N with
 *   (i+1)*m <= q_pos[b] + 1, the causal rule of the indexer (an entry
 *   exists once its block of m tokens is complete).  A query that sees no
 *   entry gets a zero output and lse = -inf.
 * norm_eps as in cskv_sparse_attend (every row is a compressed entry).
 * Errors as cskv_sparse_attend, plus INVALID_ARG for m < 1 with q_pos.
 */
size_t cskv_hca_workspace_size(int64_t B, int32_t H, int64_t N);
int cskv_hca_attend(const void* q, const void* entries, int64_t B, int32_t H, int64_t N,
                    int64_t ent_bstride, const int64_t* q_pos, int32_t m, float scale,
                    const float* sink, float norm_eps, cskv_dtype dt, void* out, float* lse,
                    void* workspace, size_t ws_bytes, void* stream);

/*
 * CSA sparse attention and HCA dense attention over MXFP4 entries
 * ("Compressed attention · CSA / HCA và hai trục nén", section 3: the V4.1
 * KV cache is FP4 with block scales).  Same results as cskv_sparse_attend
 * and cskv_hca_attend in BF16 (queries, window rows and outputs are bf16)
 * with each compressed entry given as an MXFP4 row instead: 576 elements
 * in 18 blocks of 32 (OCP Microscaling v1.0: FP4 E2M1 elements, one E8M0
 * scale 2^(X-127) per block).
 *   ent_codes [N][288] bytes: element 2j of a row in the low nibble of byte
 *     j, element 2j+1 in the high nibble.  16-byte aligned.
 *   ent_scales [N][18] bytes: the scale of elements 32b .. 32b+31.
 *   ent_bstride: rows (not elements) between the entry sets of consecutive
 *     queries, 0 for one shared context.  Other arguments and the errors
 *     are those of cskv_sparse_attend / cskv_hca_attend.
 *   workspace: at least cskv_sparse_attend_mxfp4_workspace_size(B, H, W, k)
 *     or cskv_hca_attend_mxfp4_workspace_size(B, H, N, ent_bstride > 0)
 *     bytes.  The rows a call reads (each query's selected entries, or all
 *     N entries of each context) are decoded into it as bf16 first.
 * The entries decode to bf16 exactly while every decoded value lies in
 * bf16's normal range (scale bytes 2..252 with any code, at least).
 */
size_t cskv_sparse_attend_mxfp4_workspace_size(int64_t B, int32_t H, int32_t W, int32_t k);
size_t cskv_hca_attend_mxfp4_workspace_size(int64_t B, int32_t H, int64_t N, int32_t per_sequence);
int cskv_sparse_attend_mxfp4(const void* q, const void* ent_codes, const uint8_t* ent_scales,
                             const void* window, const int32_t* idx, int64_t B, int32_t H,
                             int64_t N, int32_t W, int32_t k, int64_t ent_bstride,
                             int64_t win_bstride, int64_t win_rows, const int64_t* q_pos,
                             int64_t win_pos0, float scale, const float* sink, float norm_eps,
                             void* out, float* lse, void* workspace, size_t ws_bytes,
                             void* stream);
int cskv_hca_attend_mxfp4(const void* q, const void* ent_codes, const uint8_t* ent_scales,
                          int64_t B, int32_t H, int64_t N, int64_t ent_bstride,
                          const int64_t* q_pos, int32_t m, float scale, const float* sink,
                          float norm_eps, void* out, float* lse, void* workspace, size_t ws_bytes,
                          void* stream);

/*
 * CSA sparse attention and HCA dense attention over MXFP8 entries: the
 * compressed entries stored in FP8 with block scales ("Compressed attention
 * · CSA / HCA và hai trục nén", section 3: the compressed KV cache in
 * low-bit floating point with block scales), read as the OCP Microscaling
 * v1.0 MXFP8 format with E4M3 elements: 32 elements share one E8M0 scale
 * 2^(X-127), element value = scale * E4M3 value.  Same calls, arguments,
 * results and errors as the *_mxfp4 calls above, with
 *   ent_codes [N][576] bytes: one E4M3 code an element.  16-byte aligned.
 *   ent_scales [N][18] bytes: the scale of elements 32b .. 32b+31.
 *   workspace: the size of the matching *_mxfp4 call
 *     (cskv_sparse_attend_mxfp4_workspace_size, cskv_hca_attend_mxfp4_workspace_size):
 *     the rows a call reads are decoded into it as bf16 first.
 * The entries decode to bf16 exactly while every decoded value lies in
 * bf16's normal range.
 */
int cskv_sparse_attend_mxfp8(const void* q, const void* ent_codes, const uint8_t* ent_scales,
                             const void* window, const int32_t* idx, int64_t B, int32_t H,
                             int64_t N, int32_t W, int32_t k, int64_t ent_bstride,
                             int64_t win_bstride, int64_t win_rows, const int64_t* q_pos,
                             int64_t win_pos0, float scale, const float* sink, float norm_eps,
                             void* out, float* lse, void* workspace, size_t ws_bytes,
                             void* stream);
int cskv_hca_attend_mxfp8(const void* q, const void* ent_codes, const uint8_t* ent_scales,
                          int64_t B, int32_t H, int64_t N, int64_t ent_bstride,
                          const int64_t* q_pos, int32_t m, float scale, const float* sink,
                          float norm_eps, void* out, float* lse, void* workspace, size_t ws_bytes,
                          void* stream);

/*
 * Merge of split-KV partial results: for each (b, h) with S partial results
 * o_part[b][h][s][512] (fp32, each normalised over its own rows, no sink)
 * and lse_part[b][h][s]:  lse = ln(sum_s exp(lse_s) + exp(sink[h])),
 * out = sum_s exp(lse_s - lse) * o_s.  A split with no rows has lse_s = -inf
 * and contributes nothing; sink (nullable) as in cskv_sparse_attend.
 * out [B][H][512] in dt; lse may be NULL.
 */
int cskv_merge(const float* o_part, const float* lse_part, int64_t B, int32_t H, int32_t S,
               const float* sink, void* out, float* lse, cskv_dtype dt, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* CSKV_H */
