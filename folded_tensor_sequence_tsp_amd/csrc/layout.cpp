// Host-side sizes of the kernels' tilings and workspaces: plain C++ with no
// device code, so that the C-ABI layer and its sanitizer build (a host-only
// build of tsp_api.cpp with these sizes and recorded launches) share them.
#include "kernels.h"

namespace tsp {

bool attn_split(int64_t chunk_len, int32_t n_heads) {
  const int64_t tpc = (chunk_len + ATTN_QT - 1) / ATTN_QT;
  return chunk_len > 0 && 2 * (int64_t)n_heads * tpc < ATTN_SPLIT_BELOW;
}

int64_t attn_kv_tiles(int64_t seq_len) { return (seq_len + ATTN_BKV - 1) / ATTN_BKV; }

size_t attn_core_workspace(int64_t seq_len, int64_t chunk_len, int32_t hidden, int32_t n_heads) {
  (void)seq_len;
  if (!attn_split(chunk_len, n_heads)) return 0;
  return attn_align((size_t)2 * chunk_len * hidden * 4) + attn_align((size_t)2 * n_heads * chunk_len * 2 * 4);
}

size_t attn_bwd_ws_bytes(int64_t seq_len, int64_t chunk_len, int32_t n_heads, int32_t kv_heads, int32_t head_dim) {
  const int64_t n_kv_tiles = (seq_len + 63) / 64, tpc = (chunk_len + 63) / 64;
  const size_t kt = attn_bwd_stages_kt(head_dim) ? (size_t)kv_heads * n_kv_tiles * head_dim * 64 * 2 : 0;
  const size_t qt = attn_bwd_stages_qt(head_dim) ? (size_t)2 * n_heads * tpc * head_dim * 64 * 2 : 0;
  const size_t stats = (size_t)2 * n_heads * tpc * 256 * 4;
  return kt + 2 * qt + stats;
}

int64_t rms_norm_bwd_blocks(int64_t n) { return (n + RMS_BWD_ROWS - 1) / RMS_BWD_ROWS; }

}  // namespace tsp
