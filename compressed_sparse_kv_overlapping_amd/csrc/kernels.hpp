// Launchers of the gfx950 kernels (host side).  Each returns the HIP status
// of its launches; argument checking happens before, in api.cpp.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace cskv {

hipError_t launch_compress(int dt, const void* x, const void* z, const float* bias, int m,
                           int64_t e_begin, int64_t e_end, void* out, int64_t ld_out,
                           hipStream_t stream);
hipError_t launch_compress_fused(int dt, const void* x, const void* z, int64_t T_tokens,
                                 const float* bias_s, int ms, void* out_s, int64_t ld_s,
                                 const float* bias_l, int ml, void* out_l, int64_t ld_l, void* ws,
                                 hipStream_t stream);
size_t compress_fused_workspace_bytes(int64_t T_tokens, int ml);

struct AttendParams {
  int dt;                    // 0 fp32, 1 bf16
  const void* q;             // [B][H][576]
  const void* entries;       // [N][576] (+ b * ent_bstride)
  const void* window;        // rows of 576 (+ b * win_bstride)
  const int32_t* idx;        // [B][k] selected entries (unused when dense)
  const int64_t* q_pos;      // NULL = decode window
  int64_t B, N, ent_bstride, win_bstride, win_pos0, win_rows;
  int H, W, k;
  float scale;
  void* out;                 // [B][H][512]
  float* lse;                // [B][H] or NULL
  int dense;                 // 1: rows = all N entries, no window
  int hm;                    // dense with q_pos: entry i visible iff (i+1)*hm <= q_pos[b]+1
  const float* sink;         // [H] attention-sink logits, or NULL
  float norm_eps = -1.f;     // >= 0: queries and compressed entries normalised (unit RMS, this epsilon)
};

int attend_splits(int dt, int64_t B, int H, int64_t nslots);
size_t attend_partial_bytes(int dt, int64_t B, int H, int64_t nslots);
hipError_t launch_attend(const AttendParams& p, void* ws, hipStream_t stream);
// MX entry rows (bits 4: MXFP4 codes [.][288]; bits 8: MXFP8 codes [.][576];
// E8M0 scales [.][18]) decoded to bf16 rows of 576: dense (idx NULL) rows
// b * N + i, or gathered rows b * k + j with idx_out[b][j] = j or -1.
hipError_t launch_mx_rows(int bits, const uint8_t* codes, const uint8_t* scales, const int32_t* idx,
                          int64_t rows, int k, int64_t N, int64_t ent_bstride, void* out,
                          int32_t* idx_out, hipStream_t stream);
hipError_t launch_merge(int dt, const float* o_part, const float* lse_part, int64_t BH, int S,
                        const float* sink, int H, void* out, float* lse, hipStream_t stream);

struct TopkParams {
  int dt;                    // 0 fp32, 1 bf16, 2 fp8 e4m3, 3 MXFP4
  const void* q;             // [B][64]
  const void* keys;          // [N][64] (+ b * key_bstride elements)
  const int64_t* q_pos;      // NULL at decode
  int64_t key_bstride, B, N;
  int k, m;
  float scale;
  int32_t* out;              // [B][k]
  const uint8_t* qsc = nullptr;   // MXFP4: E8M0 scales of the queries [B][2]
  const uint8_t* ksc = nullptr;   // MXFP4: E8M0 scales of the keys [N][2]
  size_t ws_bytes = 0;            // workspace size (per-sequence keys: room to keep the scores)
};

int topk_max_k();
int64_t topk_max_entries();
size_t topk_workspace_bytes(int64_t B, int64_t N, int k);
// extra workspace with which per-sequence selections read every key once
size_t topk_stored_score_bytes(int64_t B, int64_t N);
hipError_t launch_topk(const TopkParams& p, void* ws, hipStream_t stream);

// The allocation-free calls' scratch: its size, and its device address on
// the current device (looked up once per device).
size_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(void** ptr);

}  // namespace cskv
