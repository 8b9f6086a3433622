// Recording stand-ins for the HIP kernel launches of libtsp, for the host-only
// sanitizer build of the C-ABI layer (tsp_api.cpp + layout.cpp).  Each stand-in
// checks the launch's preconditions and that every byte range the kernel would
// read or write (as the launch interface in kernels.h defines it) lies inside
// one caller buffer, then counts the launch.  Nothing is computed.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "kernels.h"
#include "registry.h"

namespace {

struct Region {
  const char* lo;
  const char* hi;
};
std::vector<Region> g_regions;
int g_launches = 0;

// Bytes of a row-major view: `rows` rows of stride `ld` elements, the last row
// `cols` elements long.
size_t span(int64_t rows, int64_t ld, int64_t cols, size_t esize) {
  if (rows <= 0 || cols <= 0) return 0;
  return (size_t)((rows - 1) * ld + cols) * esize;
}

}  // namespace

void* hc_alloc(size_t bytes) {
  void* p = aligned_alloc(256, (bytes + 255) / 256 * 256 + 256);
  if (!p) {
    fprintf(stderr, "host_check: allocation of %zu bytes failed\n", bytes);
    abort();
  }
  memset(p, 0, bytes);
  g_regions.push_back({static_cast<const char*>(p), static_cast<const char*>(p) + bytes});
  return p;
}

void hc_free_all() {
  for (const Region& r : g_regions) free(const_cast<char*>(r.lo));
  g_regions.clear();
}

void hc_need(const void* p, size_t bytes, const char* what) {
  if (bytes == 0) return;
  const char* a = static_cast<const char*>(p);
  for (const Region& r : g_regions)
    if (a >= r.lo && a + bytes <= r.hi && a + bytes >= a) return;
  fprintf(stderr, "host_check: %s: [%p, +%zu) is outside every caller buffer\n", what, p, bytes);
  abort();
}

void hc_expect(bool cond, const char* what) {
  if (!cond) {
    fprintf(stderr, "host_check: launch precondition failed: %s\n", what);
    abort();
  }
}

int hc_launches() { return g_launches; }
void hc_reset_launches() { g_launches = 0; }
void hc_count_launch() { ++g_launches; }

namespace tsp {

hipError_t launch_gemm(const GemmArgs& g, hipStream_t) {
  if (g.M <= 0) return hipSuccess;
  hc_expect(g.N_s > 0 && g.N_s % 8 == 0, "gemm: N_s a positive multiple of 8");
  hc_expect(g.K_s > 0 && g.K_s % 32 == 0, "gemm: K_s a positive multiple of 32");
  hc_expect(g.lda % 8 == 0, "gemm: lda a multiple of 8");
  hc_expect(g.n_shards >= 1 && g.k_shards >= 1 && (g.n_shards == 1 || g.k_shards == 1), "gemm: shard modes");
  hc_expect(g.k_shards <= 3 * TSP_MAX_D && g.n_shards <= TSP_MAX_D, "gemm: shard counts");
  hc_expect(g.ring_start >= 0 && (g.k_shards == 1 || g.ring_start < g.k_shards), "gemm: ring start");
  const int64_t acols = (int64_t)g.K_s * g.k_shards;
  hc_expect(g.lda >= acols, "gemm: lda covers the A columns");
  hc_need(g.A, span(g.M, g.lda, acols, 2), "gemm A");
  if (g.A_lo) hc_need(g.A_lo, span(g.M, g.lda, acols, 2), "gemm A_lo");
  for (int d = 0; d < std::max(g.n_shards, g.k_shards); ++d) hc_need(g.B[d], (size_t)g.N_s * g.K_s * 2, "gemm B shard");
  if (g.row_exp) hc_need(g.row_exp, (size_t)g.M * 4, "gemm row_exp");
  if (g.arrived) {
    hc_need(g.arrived, 4, "gemm arrival counter");
    hc_need(g.arrival_status, 4, "gemm arrival status");
    hc_expect(g.spin_limit > 0, "gemm: a bounded arrival wait");
  }
  const int64_t ncols = (int64_t)g.N_s * g.n_shards;
  switch (g.epilogue) {
    case EPI_QKV: {
      const int hs_hd = g.heads_per_shard * g.head_dim;
      const int kv_hd = (g.kv_heads_per_shard ? g.kv_heads_per_shard : g.heads_per_shard) * g.head_dim;
      const int64_t kv_ld = g.kv_ld ? g.kv_ld : g.hidden;
      hc_expect(g.N_s == hs_hd + 2 * kv_hd, "qkv: N_s = Q + K + V widths");
      hc_need(g.q_out, span(g.M, g.hidden, (int64_t)(g.shard0 + g.n_shards) * hs_hd, 2), "qkv q_out");
      const int64_t last = g.M - 1;
      int64_t max_pos = last < g.chunk_len ? g.chunk_start0 + last : g.chunk_start1 + (last - g.chunk_len);
      if (g.M > g.chunk_len) max_pos = std::max(max_pos, g.chunk_start0 + g.chunk_len - 1);
      const size_t kv = span(max_pos + 1, kv_ld, (int64_t)(g.shard0 + g.n_shards) * kv_hd, 2);
      hc_need(g.k_full, kv, "qkv k_full rows");
      hc_need(g.v_full, kv, "qkv v_full rows");
      break;
    }
    case EPI_GELU:
      hc_need(g.out, span(g.M, g.ldo, ncols, 2), "gelu out");
      break;
    case EPI_DGELU:
      hc_expect(g.n_shards == 1, "dgelu: one column block");
      hc_need(g.aux, span(g.M, g.N_s, g.N_s, 4), "dgelu aux");
      hc_need(g.out, span(g.M, g.ldo, ncols, 2), "dgelu out");
      break;
    default: {
      const size_t es = g.out_f32 ? 4 : 2;
      if (g.outs[0]) {
        if (g.rows_per_out > 0) {
          hc_expect(g.n_shards == 1, "resid: row-split outputs take one column block");
          for (int64_t k = 0; k * g.rows_per_out < g.M; ++k) {
            const int64_t rows = std::min<int64_t>(g.rows_per_out, g.M - k * g.rows_per_out);
            hc_need(g.outs[k], span(rows, g.ldo, g.N_s, es), "resid outs (row blocks)");
          }
        } else {
          for (int d = 0; d < g.n_shards; ++d) hc_need(g.outs[d], span(g.M, g.ldo, g.N_s, es), "resid outs (shards)");
        }
      } else {
        hc_need(g.out, span(g.M, g.ldo, ncols, es), "resid out");
      }
      if (g.residual) hc_need(g.residual, span(g.M, g.ldo, ncols, g.res_f32 ? 4 : 2), "resid residual");
      break;
    }
  }
  hc_count_launch();
  return hipSuccess;
}

hipError_t launch_simulate_arrival(const ArrivalCopies& c, int32_t n, uint32_t* counter, uint32_t, uint64_t,
                                   hipStream_t) {
  if (n <= 0) return hipSuccess;
  hc_expect(n <= ARRIVAL_MAX, "simulate_arrival: copies");
  hc_need(counter, 4, "simulate_arrival counter");
  for (int i = 0; i < n; ++i) {
    hc_expect(c.bytes[i] % 16 == 0, "simulate_arrival: 16-byte multiples");
    hc_need(c.src[i], c.bytes[i], "simulate_arrival src");
    hc_need(c.dst[i], c.bytes[i], "simulate_arrival dst");
  }
  hc_count_launch();
  return hipSuccess;
}

hipError_t launch_row_prep(const void* x, int32_t x_f32, int64_t n, int32_t h, int32_t* row_exp, uint16_t* x16,
                           hipStream_t) {
  if (n <= 0) return hipSuccess;
  hc_need(x, (size_t)n * h * (x_f32 ? 4 : 2), "row_prep x");
  hc_need(row_exp, (size_t)n * 4, "row_prep row_exp");
  if (x16) hc_need(x16, (size_t)n * h * 2, "row_prep x16");
  hc_count_launch();
  return hipSuccess;
}

hipError_t launch_bf16_to_f16(const uint16_t* const* src, uint16_t* dst, int32_t D, int64_t count, hipStream_t) {
  hc_expect(count % 8 == 0 && D >= 1 && D <= TSP_MAX_D, "bf16_to_f16: count % 8, D");
  for (int d = 0; d < D; ++d) hc_need(src[d], (size_t)count * 2, "bf16_to_f16 src shard");
  hc_need(dst, (size_t)D * count * 2, "bf16_to_f16 dst");
  hc_count_launch();
  return hipSuccess;
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t) {
  if (a.chunk_len <= 0) return hipSuccess;
  hc_expect(a.head_dim == 64 || a.head_dim == 128, "attention: head_dim");
  hc_expect((int64_t)a.n_heads * a.head_dim == a.hidden, "attention: hidden = heads x head_dim");
  hc_expect(a.kv_heads >= 1 && a.n_heads % a.kv_heads == 0, "attention: head groups");
  hc_expect(a.kv_ld >= a.kv_heads * a.head_dim && a.kv_ld % 8 == 0, "attention: kv_ld");
  hc_expect(a.chunk_start0 + a.chunk_len <= a.seq_len && a.chunk_start1 + a.chunk_len <= a.seq_len,
            "attention: chunks inside the sequence");
  const int64_t n = 2 * a.chunk_len;
  hc_need(a.q, (size_t)n * a.hidden * 2, "attention q");
  hc_need(a.o, (size_t)n * a.hidden * 2, "attention o");
  if (a.o_lo) hc_need(a.o_lo, (size_t)n * a.hidden * 2, "attention o_lo");
  const int64_t last_key = std::max(a.chunk_start0, a.chunk_start1) + a.chunk_len - 1;
  const size_t kv = span(last_key + 1, a.kv_ld, (int64_t)a.kv_heads * a.head_dim, 2);
  hc_need(a.k, kv, "attention k rows");
  hc_need(a.v, kv, "attention v rows");
  if (a.lse) hc_need(a.lse, (size_t)a.n_heads * n * 4, "attention lse");
  const size_t ws = attn_core_workspace(a.seq_len, a.chunk_len, a.hidden, a.n_heads);
  if (ws) hc_need(a.ws, ws, "attention workspace");
  hc_count_launch();
  return hipSuccess;
}

hipError_t launch_vt_tiles(const uint16_t* src, int64_t rows, int32_t ld, int32_t heads, int32_t head_dim,
                           uint16_t* dst, int64_t n_tiles, hipStream_t) {
  if (rows <= 0 || n_tiles <= 0) return hipSuccess;
  hc_expect(n_tiles * 64 >= rows, "vt_tiles: tiles cover the rows");
  hc_need(src, span(rows, ld, (int64_t)heads * head_dim, 2), "vt_tiles src");
  hc_need(dst, (size_t)heads * n_tiles * head_dim * 64 * 2, "vt_tiles dst");
  hc_count_launch();
  return hipSuccess;
}

hipError_t launch_zero_f32(float* p, int64_t count, hipStream_t) {
  if (count <= 0) return hipSuccess;
  hc_need(p, (size_t)count * 4, "zero_f32");
  hc_count_launch();
  return hipSuccess;
}

hipError_t launch_f32_to_bf16(const float* src, int64_t R, int64_t C, int64_t ld_in, uint16_t* dst, int64_t ld_out,
                              hipStream_t) {
  if (R <= 0) return hipSuccess;
  hc_expect(C % 8 == 0, "f32_to_bf16: C % 8");
  hc_need(src, span(R, ld_in, C, 4), "f32_to_bf16 src");
  hc_need(dst, span(R, ld_out, C, 2), "f32_to_bf16 dst");
  hc_count_launch();
  return hipSuccess;
}

hipError_t launch_attention_backward(const AttnBwdArgs& a, hipStream_t) {
  if (a.chunk_len <= 0) return hipSuccess;
  hc_expect(a.head_dim == 64 || a.head_dim == 128, "attn bwd: head_dim");
  hc_expect(a.kv_heads >= 1 && a.n_heads % a.kv_heads == 0 && a.kv_ld >= a.kv_heads * a.head_dim,
            "attn bwd: K/V heads");
  const int64_t n = 2 * a.chunk_len;
  for (const void* p : {(const void*)a.q, (const void*)a.o, (const void*)a.dout})
    hc_need(p, (size_t)n * a.hidden * 2, "attn bwd q/o/dout");
  if (a.o_lo) hc_need(a.o_lo, (size_t)n * a.hidden * 2, "attn bwd o_lo");
  hc_need(a.lse, (size_t)a.n_heads * n * 4, "attn bwd lse");
  hc_need(a.dq, (size_t)n * a.hidden * 4, "attn bwd dq");
  hc_need(a.k, span(a.seq_len, a.kv_ld, (int64_t)a.kv_heads * a.head_dim, 2), "attn bwd k");
  hc_need(a.v, span(a.seq_len, a.kv_ld, (int64_t)a.kv_heads * a.head_dim, 2), "attn bwd v");
  hc_need(a.dk, (size_t)a.seq_len * a.kv_ld * 4, "attn bwd dk");
  hc_need(a.dv, (size_t)a.seq_len * a.kv_ld * 4, "attn bwd dv");
  hc_expect(a.n_kv_tiles * 64 >= a.seq_len && a.tpc * 64 >= a.chunk_len, "attn bwd: tile counts");
  if (attn_bwd_stages_kt(a.head_dim))
    hc_need(a.kt, (size_t)a.kv_heads * a.n_kv_tiles * a.head_dim * 64 * 2, "attn bwd K^T tiles");
  if (attn_bwd_stages_qt(a.head_dim)) {
    hc_need(a.qt, (size_t)2 * a.n_heads * a.tpc * a.head_dim * 64 * 2, "attn bwd Q^T tiles");
    hc_need(a.dot, (size_t)2 * a.n_heads * a.tpc * a.head_dim * 64 * 2, "attn bwd dO^T tiles");
  }
  hc_need(a.stats, (size_t)2 * a.n_heads * a.tpc * 256 * 4, "attn bwd stats");
  hc_count_launch();
  return hipSuccess;
}

hipError_t launch_rms_norm(const uint16_t* x, const uint16_t* gain, int64_t n, int32_t h, float, uint16_t* y,
                           hipStream_t) {
  if (n <= 0) return hipSuccess;
  hc_expect(h % 8 == 0, "rms_norm: h % 8");
  hc_need(x, (size_t)n * h * 2, "rms_norm x");
  hc_need(y, (size_t)n * h * 2, "rms_norm y");
  hc_need(gain, (size_t)h * 2, "rms_norm gain");
  hc_count_launch();
  return hipSuccess;
}

hipError_t launch_rope(void* x, int32_t x_f32, int32_t, int64_t n_rows, int64_t ld, int32_t n_heads,
                       int32_t head_dim, double, int64_t chunk_len, int64_t start0, int64_t start1,
                       int32_t at_global, hipStream_t) {
  if (n_rows <= 0) return hipSuccess;
  hc_expect(n_rows <= 2 * chunk_len, "rope: rows within the two chunks");
  const int64_t last = n_rows - 1;
  int64_t max_row = last;
  if (at_global) {
    max_row = last < chunk_len ? start0 + last : start1 + (last - chunk_len);
    if (n_rows > chunk_len) max_row = std::max(max_row, start0 + chunk_len - 1);
  }
  hc_need(x, span(max_row + 1, ld, (int64_t)n_heads * head_dim, x_f32 ? 4 : 2), "rope rows");
  hc_count_launch();
  return hipSuccess;
}

hipError_t launch_rms_norm_backward(const uint16_t* x, const uint16_t* gain, const uint16_t* dy, int64_t n,
                                    int32_t h, float, uint16_t* dx, float* dgain, float* partial, hipStream_t) {
  hc_expect(h % 8 == 0 && h <= 8192, "rms_norm_backward: h");
  hc_need(gain, (size_t)h * 2, "rms bwd gain");
  hc_need(dgain, (size_t)h * 4, "rms bwd dgain");
  if (n > 0) {
    hc_need(x, (size_t)n * h * 2, "rms bwd x");
    hc_need(dy, (size_t)n * h * 2, "rms bwd dy");
    hc_need(dx, (size_t)n * h * 2, "rms bwd dx");
    hc_need(partial, (size_t)rms_norm_bwd_blocks(n) * h * 4, "rms bwd partial");
  }
  hc_count_launch();
  return hipSuccess;
}

hipError_t launch_transpose(const void* src, int32_t src_f32, int32_t, int64_t R, int64_t C, int64_t ld_in,
                            uint16_t* dst, int64_t ld_out, hipStream_t) {
  hc_expect(C % 64 == 0 && ld_out % 64 == 0 && ld_out >= R, "transpose: C, ld_out");
  if (R > 0) hc_need(src, span(R, ld_in, C, src_f32 ? 4 : 2), "transpose src");
  hc_need(dst, (size_t)C * ld_out * 2, "transpose dst");
  hc_count_launch();
  return hipSuccess;
}

}  // namespace tsp
