// C-ABI entry points of libcskv: argument validation, launch configuration,
// workspace carving and the per-thread error message.  Every check runs
// before any launch, so a rejected call writes nothing.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/cskv.h"
#include "kernels.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  try {                                    // no exception may leave a C entry point
    g_last_error = buf;
  } catch (...) {
    g_last_error.clear();
  }
  return code;
}

int ok() {
  g_last_error.clear();
  return CSKV_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(CSKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t kD = 512;

}  // namespace

extern "C" {

int cskv_version(void) { return CSKV_VERSION; }

const char* cskv_status_string(int status) {
  switch (status) {
    case CSKV_OK: return "ok";
    case CSKV_ERR_INVALID_ARG: return "invalid argument";
    case CSKV_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case CSKV_ERR_WORKSPACE: return "workspace missing or too small";
    case CSKV_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* cskv_last_error(void) { return g_last_error.c_str(); }

int cskv_compress(const void* raw_kv, const void* score_logits, const float* pos_bias, int64_t T,
                  int32_t m, int64_t entry_begin, int64_t entry_end, void* out, int64_t ld_out,
                  cskv_dtype dt, void* stream) {
  if (T < 0 || m < 1) return fail(CSKV_ERR_INVALID_ARG, "cskv_compress: T=%lld m=%d", (long long)T, m);
  const int64_t N = T / m;
  if (entry_begin < 0 || entry_end < entry_begin || entry_end > N)
    return fail(CSKV_ERR_INVALID_ARG, "cskv_compress: entry range [%lld, %lld) outside [0, %lld]",
                (long long)entry_begin, (long long)entry_end, (long long)N);
  if (ld_out < kD || ld_out % 8 != 0)
    return fail(CSKV_ERR_INVALID_ARG, "cskv_compress: ld_out=%lld (need >= 512, multiple of 8)",
                (long long)ld_out);
  if (dt != CSKV_F32 && dt != CSKV_BF16)
    return fail(CSKV_ERR_UNSUPPORTED, "cskv_compress: dtype %d (F32 or BF16)", (int)dt);
  if (entry_end == entry_begin) return ok();   // nothing to write: pointers are not used
  if (!raw_kv || !score_logits || !pos_bias || !out)
    return fail(CSKV_ERR_INVALID_ARG, "cskv_compress: null pointer");
  if (!aligned16(raw_kv) || !aligned16(score_logits) || !aligned16(pos_bias) || !aligned16(out))
    return fail(CSKV_ERR_INVALID_ARG, "cskv_compress: tensors must be 16-byte aligned");
  return hip_status(cskv::launch_compress((int)dt, raw_kv, score_logits, pos_bias, m, entry_begin,
                                          entry_end, out, ld_out, (hipStream_t)stream),
                    "cskv_compress");
}

size_t cskv_compress2_workspace_size(int64_t T, int32_t m_large) {
  if (T < 0 || m_large < 1 || m_large > 65536) return 0;
  return cskv::compress_fused_workspace_bytes(T, m_large);
}

int cskv_compress2(const void* raw_kv, const void* score_logits, int64_t T,
                   const float* bias_small, int32_t m_small, void* out_small, int64_t ld_small,
                   const float* bias_large, int32_t m_large, void* out_large, int64_t ld_large,
                   cskv_dtype dt, void* workspace, size_t ws_bytes, void* stream) {
  if (T < 0 || m_small < 1 || m_large < 1)
    return fail(CSKV_ERR_INVALID_ARG, "cskv_compress2: T=%lld m_small=%d m_large=%d", (long long)T,
                m_small, m_large);
  if (m_large % m_small != 0 || m_large == m_small)
    return fail(CSKV_ERR_INVALID_ARG, "cskv_compress2: m_large=%d must be a multiple (> 1) of m_small=%d",
                m_large, m_small);
  if (ld_small < kD || ld_small % 8 != 0 || ld_large < kD || ld_large % 8 != 0)
    return fail(CSKV_ERR_INVALID_ARG, "cskv_compress2: ld_small=%lld ld_large=%lld", (long long)ld_small,
                (long long)ld_large);
  if (m_small > 4 || m_large > 65536)
    return fail(CSKV_ERR_UNSUPPORTED, "cskv_compress2: m_small=%d (max 4) m_large=%d (max 65536)",
                m_small, m_large);
  if (dt != CSKV_F32 && dt != CSKV_BF16)
    return fail(CSKV_ERR_UNSUPPORTED, "cskv_compress2: dtype %d (F32 or BF16)", (int)dt);
  if (T / m_small == 0) return ok();           // nothing to write
  const bool large = T / m_large > 0;           // the large-scale pointers are used only then
  if (!raw_kv || !score_logits || !bias_small || !out_small || (large && (!bias_large || !out_large)))
    return fail(CSKV_ERR_INVALID_ARG, "cskv_compress2: null pointer");
  if (!aligned16(raw_kv) || !aligned16(score_logits) || !aligned16(bias_small) ||
      !aligned16(out_small) || (large && (!aligned16(bias_large) || !aligned16(out_large))))
    return fail(CSKV_ERR_INVALID_ARG, "cskv_compress2: tensors must be 16-byte aligned");
  const size_t need = cskv::compress_fused_workspace_bytes(T, m_large);
  if (!workspace || ws_bytes < need || !aligned16(workspace))
    return fail(CSKV_ERR_WORKSPACE, "cskv_compress2: workspace %zu bytes, need %zu", ws_bytes, need);
  return hip_status(cskv::launch_compress_fused((int)dt, raw_kv, score_logits, T, bias_small, m_small,
                                                out_small, ld_small, bias_large, m_large, out_large,
                                                ld_large, workspace, (hipStream_t)stream),
                    "cskv_compress2");
}

size_t cskv_index_topk_workspace_size(int64_t B, int64_t N, int32_t k) {
  if (B < 1 || N < 1 || k < 1) return 0;
  return cskv::topk_workspace_bytes(B, N, k);
}

size_t cskv_index_topk_per_seq_workspace_size(int64_t B, int64_t N, int32_t k) {
  if (B < 1 || N < 1 || k < 1) return 0;
  return cskv::topk_workspace_bytes(B, N, k) + cskv::topk_stored_score_bytes(B, N);
}

static int check_topk(const char* fn, const void* q_idx, const void* idx_keys, int64_t B, int64_t N,
                      int32_t k, int64_t key_bstride, const int64_t* q_pos, int32_t m,
                      float idx_scale, cskv_dtype idx_dt, const int32_t* idx_out) {
  if (!q_idx || !idx_keys || !idx_out) return fail(CSKV_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (B < 1 || N < 1 || k < 1 || key_bstride < 0)
    return fail(CSKV_ERR_INVALID_ARG, "%s: B=%lld N=%lld k=%d key_bstride=%lld", fn, (long long)B,
                (long long)N, k, (long long)key_bstride);
  if (q_pos && m < 1) return fail(CSKV_ERR_INVALID_ARG, "%s: m=%d with q_pos", fn, m);
  if (!(idx_scale > 0.f) || idx_scale > 3.0e38f)
    return fail(CSKV_ERR_INVALID_ARG, "%s: idx_scale must be positive and finite", fn);
  if (idx_dt != CSKV_F32 && idx_dt != CSKV_BF16 && idx_dt != CSKV_FP8_E4M3)
    return fail(CSKV_ERR_UNSUPPORTED, "%s: idx dtype %d", fn, (int)idx_dt);
  if (k > cskv::topk_max_k())
    return fail(CSKV_ERR_UNSUPPORTED, "%s: k=%d > %d", fn, k, cskv::topk_max_k());
  if (N > cskv::topk_max_entries() || B > (int64_t)1 << 30)
    return fail(CSKV_ERR_UNSUPPORTED, "%s: N=%lld (max %lld) B=%lld", fn, (long long)N,
                (long long)cskv::topk_max_entries(), (long long)B);
  if (key_bstride % 64 != 0) return fail(CSKV_ERR_INVALID_ARG, "%s: key_bstride %% 64 != 0", fn);
  if (!aligned16(q_idx) || !aligned16(idx_keys))
    return fail(CSKV_ERR_INVALID_ARG, "%s: tensors must be 16-byte aligned", fn);
  return CSKV_OK;
}

int cskv_index_topk(const void* q_idx, const void* idx_keys, int64_t B, int64_t N, int32_t k,
                    int64_t key_bstride, const int64_t* q_pos, int32_t m, float idx_scale,
                    cskv_dtype idx_dt, int32_t* idx_out, void* workspace, size_t ws_bytes,
                    void* stream) {
  int st = check_topk("cskv_index_topk", q_idx, idx_keys, B, N, k, key_bstride, q_pos, m,
                      idx_scale, idx_dt, idx_out);
  if (st) return st;
  const size_t need = cskv::topk_workspace_bytes(B, N, k);
  if (!workspace || ws_bytes < need || !aligned16(workspace))
    return fail(CSKV_ERR_WORKSPACE, "cskv_index_topk: workspace %zu bytes, need %zu", ws_bytes, need);
  cskv::TopkParams p{(int)idx_dt, q_idx, idx_keys, q_pos, key_bstride, B, N, k, m, idx_scale, idx_out};
  p.ws_bytes = ws_bytes;
  return hip_status(cskv::launch_topk(p, workspace, (hipStream_t)stream), "cskv_index_topk");
}

size_t cskv_index_topk_noalloc_max_bytes(void) { return cskv::noalloc_scratch_bytes(); }

int cskv_index_topk_noalloc(const void* q_idx, const void* idx_keys, int64_t B, int64_t N, int32_t k,
                            int64_t key_bstride, const int64_t* q_pos, int32_t m, float idx_scale,
                            cskv_dtype idx_dt, int32_t* idx_out, void* stream) {
  const char* fn = "cskv_index_topk_noalloc";
  int st = check_topk(fn, q_idx, idx_keys, B, N, k, key_bstride, q_pos, m, idx_scale, idx_dt,
                      idx_out);
  if (st) return st;
  const size_t need = cskv::topk_workspace_bytes(B, N, k);
  const size_t have = cskv::noalloc_scratch_bytes();
  if (need > have)
    return fail(CSKV_ERR_UNSUPPORTED,
                "%s: this selection needs %zu bytes of scratch; the allocation-free call has %zu "
                "(use cskv_index_topk with a workspace)", fn, need, have);
  void* ws = nullptr;
  hipError_t e = cskv::noalloc_scratch(&ws);
  if (e != hipSuccess) return hip_status(e, "cskv_index_topk_noalloc (scratch address)");
  cskv::TopkParams p{(int)idx_dt, q_idx, idx_keys, q_pos, key_bstride, B, N, k, m, idx_scale, idx_out};
  p.ws_bytes = have;
  return hip_status(cskv::launch_topk(p, ws, (hipStream_t)stream), fn);
}

int cskv_index_topk_mxfp4(const void* q_codes, const uint8_t* q_scales, const void* key_codes,
                          const uint8_t* key_scales, int64_t B, int64_t N, int32_t k,
                          int64_t key_bstride, const int64_t* q_pos, int32_t m, float idx_scale,
                          int32_t* idx_out, void* workspace, size_t ws_bytes, void* stream) {
  const char* fn = "cskv_index_topk_mxfp4";
  if (!q_scales || !key_scales) return fail(CSKV_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (key_bstride < 0 || key_bstride > ((int64_t)1 << 40))
    return fail(CSKV_ERR_INVALID_ARG, "%s: key_bstride=%lld", fn, (long long)key_bstride);
  // rows are 64 elements: the element stride the shared checks expect
  int st = check_topk(fn, q_codes, key_codes, B, N, k, key_bstride * 64, q_pos, m, idx_scale,
                      CSKV_BF16, idx_out);
  if (st) return st;
  if ((reinterpret_cast<uintptr_t>(q_scales) | reinterpret_cast<uintptr_t>(key_scales)) & 1u)
    return fail(CSKV_ERR_INVALID_ARG, "%s: scale arrays must be 2-byte aligned", fn);
  const size_t need = cskv::topk_workspace_bytes(B, N, k);
  if (!workspace || ws_bytes < need || !aligned16(workspace))
    return fail(CSKV_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn, ws_bytes, need);
  cskv::TopkParams p{3, q_codes, key_codes, q_pos, key_bstride * 64, B, N, k, m, idx_scale, idx_out,
                     q_scales, key_scales};
  p.ws_bytes = ws_bytes;
  return hip_status(cskv::launch_topk(p, workspace, (hipStream_t)stream), fn);
}

size_t cskv_attend_workspace_size(int64_t B, int32_t H, int64_t rows_per_query) {
  if (B < 1 || H < 1 || rows_per_query < 0) return 0;
  // the larger of the fp32 and bf16 layouts, so one size serves both
  size_t a = cskv::attend_partial_bytes(0, B, H, rows_per_query);
  size_t b = cskv::attend_partial_bytes(1, B, H, rows_per_query);
  return a > b ? a : b;
}

static int check_attend(const char* fn, const void* q, const void* entries, const void* window,
                        int64_t B, int32_t H, int64_t N, int32_t W, int32_t k, int64_t ent_bstride,
                        int64_t win_bstride, int64_t win_rows, cskv_dtype dt, const void* out,
                        float scale, float norm_eps) {
  if (!q || !entries || !out) return fail(CSKV_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (!(scale >= 0.f) || scale > 3.0e38f)
    return fail(CSKV_ERR_INVALID_ARG, "%s: scale must be non-negative and finite", fn);
  if (norm_eps != norm_eps || norm_eps > 3.0e38f)
    return fail(CSKV_ERR_INVALID_ARG, "%s: norm_eps must be finite (negative: no normalisation)", fn);
  if (W > 0 && !window) return fail(CSKV_ERR_INVALID_ARG, "%s: W=%d without a window", fn, W);
  if (B < 1 || H < 1 || N < 0 || W < 0 || k < 0 || ent_bstride < 0 || win_bstride < 0 ||
      win_rows < 0)
    return fail(CSKV_ERR_INVALID_ARG, "%s: B=%lld H=%d N=%lld W=%d k=%d", fn, (long long)B, H,
                (long long)N, W, k);
  if (dt != CSKV_F32 && dt != CSKV_BF16)
    return fail(CSKV_ERR_UNSUPPORTED, "%s: dtype %d (F32 or BF16)", fn, (int)dt);
  if (N > (int64_t)1 << 31 || (int64_t)k + W > (int64_t)1 << 30 || B > (int64_t)1 << 30)
    return fail(CSKV_ERR_UNSUPPORTED, "%s: sizes too large", fn);
  if (ent_bstride % 8 != 0 || win_bstride % 8 != 0)
    return fail(CSKV_ERR_INVALID_ARG, "%s: batch strides must be multiples of 8", fn);
  if (!aligned16(q) || !aligned16(entries) || (window && !aligned16(window)) || !aligned16(out))
    return fail(CSKV_ERR_INVALID_ARG, "%s: tensors must be 16-byte aligned", fn);
  return CSKV_OK;
}

int cskv_sparse_attend(const void* q, const void* entries, const void* window, const int32_t* idx,
                       int64_t B, int32_t H, int64_t N, int32_t W, int32_t k, int64_t ent_bstride,
                       int64_t win_bstride, int64_t win_rows, const int64_t* q_pos,
                       int64_t win_pos0, float scale, const float* sink, float norm_eps,
                       cskv_dtype dt, void* out, float* lse, void* workspace, size_t ws_bytes,
                       void* stream) {
  int st = check_attend("cskv_sparse_attend", q, entries, window, B, H, N, W, k, ent_bstride,
                        win_bstride, win_rows, dt, out, scale, norm_eps);
  if (st) return st;
  if (k > 0 && !idx) return fail(CSKV_ERR_INVALID_ARG, "cskv_sparse_attend: null idx");
  if (!q_pos && W > win_rows)
    return fail(CSKV_ERR_INVALID_ARG, "cskv_sparse_attend: W=%d > window rows %lld", W,
                (long long)win_rows);
  const size_t need = cskv::attend_partial_bytes((int)dt, B, H, (int64_t)k + W);
  if (need && (!workspace || ws_bytes < need || !aligned16(workspace)))
    return fail(CSKV_ERR_WORKSPACE, "cskv_sparse_attend: workspace %zu bytes, need %zu", ws_bytes,
                need);
  cskv::AttendParams p{(int)dt, q, entries, window, idx, q_pos, B, N, ent_bstride, win_bstride,
                       win_pos0, win_rows, H, W, k, scale, out, lse, 0, 0, sink, norm_eps};
  return hip_status(cskv::launch_attend(p, workspace, (hipStream_t)stream), "cskv_sparse_attend");
}

size_t cskv_csa_workspace_size(int64_t B, int32_t H, int64_t N, int32_t W, int32_t k) {
  if (B < 1 || H < 1 || N < 1 || k < 1 || W < 0) return 0;
  return cskv::topk_workspace_bytes(B, N, k) + 256 +
         cskv_attend_workspace_size(B, H, (int64_t)k + W);
}

int cskv_csa_attend(const void* q, const void* q_idx, const void* entries, const void* idx_keys,
                    const void* window, int64_t B, int32_t H, int64_t N, int32_t W, int32_t k,
                    int32_t m, int64_t ent_bstride, int64_t key_bstride, int64_t win_bstride,
                    int64_t win_rows, const int64_t* q_pos, int64_t win_pos0, float scale,
                    const float* sink, float norm_eps, float idx_scale, cskv_dtype dt,
                    cskv_dtype idx_dt, void* out, float* lse, int32_t* idx_out, void* workspace,
                    size_t ws_bytes, void* stream) {
  int st = check_topk("cskv_csa_attend", q_idx, idx_keys, B, N, k, key_bstride, q_pos, m,
                      idx_scale, idx_dt, idx_out);
  if (st) return st;
  st = check_attend("cskv_csa_attend", q, entries, window, B, H, N, W, k, ent_bstride, win_bstride,
                    win_rows, dt, out, scale, norm_eps);
  if (st) return st;
  if (!q_pos && W > win_rows)
    return fail(CSKV_ERR_INVALID_ARG, "cskv_csa_attend: W=%d > window rows %lld", W,
                (long long)win_rows);
  const size_t need = cskv_csa_workspace_size(B, H, N, W, k);
  if (!workspace || ws_bytes < need || !aligned16(workspace))
    return fail(CSKV_ERR_WORKSPACE, "cskv_csa_attend: workspace %zu bytes, need %zu", ws_bytes, need);
  const size_t topk_bytes = (cskv::topk_workspace_bytes(B, N, k) + 255) / 256 * 256;
  cskv::TopkParams tp{(int)idx_dt, q_idx, idx_keys, q_pos, key_bstride, B, N, k, m, idx_scale,
                      idx_out};
  hipError_t e = cskv::launch_topk(tp, workspace, (hipStream_t)stream);
  if (e != hipSuccess) return hip_status(e, "cskv_csa_attend (top-k)");
  cskv::AttendParams ap{(int)dt, q, entries, window, idx_out, q_pos, B, N, ent_bstride,
                        win_bstride, win_pos0, win_rows, H, W, k, scale, out, lse, 0, 0, sink,
                        norm_eps};
  return hip_status(cskv::launch_attend(ap, (char*)workspace + topk_bytes, (hipStream_t)stream),
                    "cskv_csa_attend (attention)");
}

size_t cskv_hca_workspace_size(int64_t B, int32_t H, int64_t N) {
  if (B < 1 || H < 1 || N < 0) return 0;
  return cskv_attend_workspace_size(B, H, N);
}

int cskv_hca_attend(const void* q, const void* entries, int64_t B, int32_t H, int64_t N,
                    int64_t ent_bstride, const int64_t* q_pos, int32_t m, float scale,
                    const float* sink, float norm_eps, cskv_dtype dt, void* out, float* lse,
                    void* workspace, size_t ws_bytes, void* stream) {
  int st = check_attend("cskv_hca_attend", q, entries, nullptr, B, H, N, 0, 0, ent_bstride, 0, 0,
                        dt, out, scale, norm_eps);
  if (st) return st;
  if (q_pos && m < 1) return fail(CSKV_ERR_INVALID_ARG, "cskv_hca_attend: m=%d with q_pos", m);
  const size_t need = cskv::attend_partial_bytes((int)dt, B, H, N);
  if (need && (!workspace || ws_bytes < need || !aligned16(workspace)))
    return fail(CSKV_ERR_WORKSPACE, "cskv_hca_attend: workspace %zu bytes, need %zu", ws_bytes, need);
  cskv::AttendParams p{(int)dt, q, entries, nullptr, nullptr, q_pos, B, N, ent_bstride, 0, 0, 0,
                       H, 0, 0, scale, out, lse, 1, q_pos ? m : 0, sink, norm_eps};
  return hip_status(cskv::launch_attend(p, workspace, (hipStream_t)stream), "cskv_hca_attend");
}

// MX entries: the codes and scales of row i of sequence b start at
// (b * ent_bstride + i) * 288 (MXFP4) or * 576 (MXFP8) and * 18 bytes.  The
// rows an attention call reads are first decoded to bf16 rows in the
// workspace (each row once: the
// selected rows of every query, or all rows for dense attention), then the
// bf16 attention kernels run on them.  Workspace: [partials][bf16 rows][row
// table].
static int check_mxfp4_entries(const char* fn, const void* codes, const uint8_t* scales,
                               int64_t ent_bstride) {
  if (!codes || !scales) return fail(CSKV_ERR_INVALID_ARG, "%s: null entry pointer", fn);
  if (ent_bstride < 0 || ent_bstride > ((int64_t)1 << 40))
    return fail(CSKV_ERR_INVALID_ARG, "%s: ent_bstride=%lld", fn, (long long)ent_bstride);
  if (!aligned16(codes)) return fail(CSKV_ERR_INVALID_ARG, "%s: entry codes must be 16-byte aligned", fn);
  return CSKV_OK;
}

static size_t round256(size_t x) { return (x + 255) / 256 * 256; }

size_t cskv_sparse_attend_mxfp4_workspace_size(int64_t B, int32_t H, int32_t W, int32_t k) {
  if (B < 1 || H < 1 || W < 0 || k < 0) return 0;
  return round256(cskv::attend_partial_bytes(1, B, H, (int64_t)k + W)) +
         round256((size_t)B * k * 576 * 2) + round256((size_t)B * k * 4);
}

size_t cskv_hca_attend_mxfp4_workspace_size(int64_t B, int32_t H, int64_t N, int32_t per_sequence) {
  if (B < 1 || H < 1 || N < 0) return 0;
  return round256(cskv::attend_partial_bytes(1, B, H, N)) +
         round256((size_t)(per_sequence ? B : 1) * N * 576 * 2);
}

// MX entries (bits 4: MXFP4, 288 code bytes a row; bits 8: MXFP8 with E4M3
// elements, 576 code bytes a row; 18 E8M0 scale bytes a row either way):
// the rows a call reads are decoded to bf16 rows in the workspace first,
// then the bf16 attention kernels run on them.
static int sparse_attend_mx(const char* fn, int bits, const void* q, const void* ent_codes,
                            const uint8_t* ent_scales, const void* window, const int32_t* idx,
                            int64_t B, int32_t H, int64_t N, int32_t W, int32_t k,
                            int64_t ent_bstride, int64_t win_bstride, int64_t win_rows,
                            const int64_t* q_pos, int64_t win_pos0, float scale, const float* sink,
                            float norm_eps, void* out, float* lse, void* workspace, size_t ws_bytes,
                            void* stream) {
  int st = check_mxfp4_entries(fn, ent_codes, ent_scales, ent_bstride);
  if (st) return st;
  st = check_attend(fn, q, ent_codes, window, B, H, N, W, k, ent_bstride * 576, win_bstride,
                    win_rows, CSKV_BF16, out, scale, norm_eps);
  if (st) return st;
  if (k > 0 && !idx) return fail(CSKV_ERR_INVALID_ARG, "%s: null idx", fn);
  if (!q_pos && W > win_rows)
    return fail(CSKV_ERR_INVALID_ARG, "%s: W=%d > window rows %lld", fn, W, (long long)win_rows);
  const size_t need = cskv_sparse_attend_mxfp4_workspace_size(B, H, W, k);
  if (!workspace || ws_bytes < need || !aligned16(workspace))
    return fail(CSKV_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn, ws_bytes, need);
  char* w = (char*)workspace;
  char* rows = w + round256(cskv::attend_partial_bytes(1, B, H, (int64_t)k + W));
  int32_t* sel = (int32_t*)(rows + round256((size_t)B * k * 576 * 2));
  hipError_t e = cskv::launch_mx_rows(bits, (const uint8_t*)ent_codes, ent_scales, idx, B * k, k, N,
                                      ent_bstride, rows, sel, (hipStream_t)stream);
  if (e != hipSuccess) return hip_status(e, fn);
  cskv::AttendParams p{1, q, rows, window, sel, q_pos, B, k, (int64_t)k * 576, win_bstride,
                       win_pos0, win_rows, H, W, k, scale, out, lse, 0, 0, sink, norm_eps};
  return hip_status(cskv::launch_attend(p, workspace, (hipStream_t)stream), fn);
}

static int hca_attend_mx(const char* fn, int bits, const void* q, const void* ent_codes,
                         const uint8_t* ent_scales, int64_t B, int32_t H, int64_t N,
                         int64_t ent_bstride, const int64_t* q_pos, int32_t m, float scale,
                         const float* sink, float norm_eps, void* out, float* lse, void* workspace,
                         size_t ws_bytes, void* stream) {
  int st = check_mxfp4_entries(fn, ent_codes, ent_scales, ent_bstride);
  if (st) return st;
  st = check_attend(fn, q, ent_codes, nullptr, B, H, N, 0, 0, ent_bstride * 576, 0, 0, CSKV_BF16,
                    out, scale, norm_eps);
  if (st) return st;
  if (q_pos && m < 1) return fail(CSKV_ERR_INVALID_ARG, "%s: m=%d with q_pos", fn, m);
  const bool per_seq = ent_bstride > 0;
  const size_t need = cskv_hca_attend_mxfp4_workspace_size(B, H, N, per_seq);
  if (!workspace || ws_bytes < need || !aligned16(workspace))
    return fail(CSKV_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn, ws_bytes, need);
  char* rows = (char*)workspace + round256(cskv::attend_partial_bytes(1, B, H, N));
  hipError_t e = cskv::launch_mx_rows(bits, (const uint8_t*)ent_codes, ent_scales, nullptr,
                                      (per_seq ? B : 1) * N, 0, N, ent_bstride, rows, nullptr,
                                      (hipStream_t)stream);
  if (e != hipSuccess) return hip_status(e, fn);
  cskv::AttendParams p{1, q, rows, nullptr, nullptr, q_pos, B, N, per_seq ? N * 576 : 0, 0, 0, 0,
                       H, 0, 0, scale, out, lse, 1, q_pos ? m : 0, sink, norm_eps};
  return hip_status(cskv::launch_attend(p, workspace, (hipStream_t)stream), fn);
}

int cskv_sparse_attend_mxfp4(const void* q, const void* ent_codes, const uint8_t* ent_scales,
                             const void* window, const int32_t* idx, int64_t B, int32_t H,
                             int64_t N, int32_t W, int32_t k, int64_t ent_bstride,
                             int64_t win_bstride, int64_t win_rows, const int64_t* q_pos,
                             int64_t win_pos0, float scale, const float* sink, float norm_eps,
                             void* out, float* lse, void* workspace, size_t ws_bytes,
                             void* stream) {
  return sparse_attend_mx("cskv_sparse_attend_mxfp4", 4, q, ent_codes, ent_scales, window, idx, B,
                          H, N, W, k, ent_bstride, win_bstride, win_rows, q_pos, win_pos0, scale,
                          sink, norm_eps, out, lse, workspace, ws_bytes, stream);
}

int cskv_hca_attend_mxfp4(const void* q, const void* ent_codes, const uint8_t* ent_scales,
                          int64_t B, int32_t H, int64_t N, int64_t ent_bstride,
                          const int64_t* q_pos, int32_t m, float scale, const float* sink,
                          float norm_eps, void* out, float* lse, void* workspace, size_t ws_bytes,
                          void* stream) {
  return hca_attend_mx("cskv_hca_attend_mxfp4", 4, q, ent_codes, ent_scales, B, H, N, ent_bstride,
                       q_pos, m, scale, sink, norm_eps, out, lse, workspace, ws_bytes, stream);
}

int cskv_sparse_attend_mxfp8(const void* q, const void* ent_codes, const uint8_t* ent_scales,
                             const void* window, const int32_t* idx, int64_t B, int32_t H,
                             int64_t N, int32_t W, int32_t k, int64_t ent_bstride,
                             int64_t win_bstride, int64_t win_rows, const int64_t* q_pos,
                             int64_t win_pos0, float scale, const float* sink, float norm_eps,
                             void* out, float* lse, void* workspace, size_t ws_bytes,
                             void* stream) {
  return sparse_attend_mx("cskv_sparse_attend_mxfp8", 8, q, ent_codes, ent_scales, window, idx, B,
                          H, N, W, k, ent_bstride, win_bstride, win_rows, q_pos, win_pos0, scale,
                          sink, norm_eps, out, lse, workspace, ws_bytes, stream);
}

int cskv_hca_attend_mxfp8(const void* q, const void* ent_codes, const uint8_t* ent_scales,
                          int64_t B, int32_t H, int64_t N, int64_t ent_bstride,
                          const int64_t* q_pos, int32_t m, float scale, const float* sink,
                          float norm_eps, void* out, float* lse, void* workspace, size_t ws_bytes,
                          void* stream) {
  return hca_attend_mx("cskv_hca_attend_mxfp8", 8, q, ent_codes, ent_scales, B, H, N, ent_bstride,
                       q_pos, m, scale, sink, norm_eps, out, lse, workspace, ws_bytes, stream);
}

int cskv_merge(const float* o_part, const float* lse_part, int64_t B, int32_t H, int32_t S,
               const float* sink, void* out, float* lse, cskv_dtype dt, void* stream) {
  if (!o_part || !lse_part || !out) return fail(CSKV_ERR_INVALID_ARG, "cskv_merge: null pointer");
  if (B < 1 || H < 1 || S < 1) return fail(CSKV_ERR_INVALID_ARG, "cskv_merge: B=%lld H=%d S=%d",
                                           (long long)B, H, S);
  if (dt != CSKV_F32 && dt != CSKV_BF16)
    return fail(CSKV_ERR_UNSUPPORTED, "cskv_merge: dtype %d (F32 or BF16)", (int)dt);
  if (!aligned16(o_part) || !aligned16(out))
    return fail(CSKV_ERR_INVALID_ARG, "cskv_merge: tensors must be 16-byte aligned");
  return hip_status(cskv::launch_merge((int)dt, o_part, lse_part, B * H, S, sink, H, out, lse,
                                       (hipStream_t)stream),
                    "cskv_merge");
}

}  // extern "C"
