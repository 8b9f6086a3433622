// C-ABI entry points of libtsp: zigzag planner, argument validation and the
// composition of the rank-share layer out of the HIP kernels.  Every check runs
// before the first launch, so an error status means nothing was enqueued.
#include <string.h>

#include <functional>

#include "kernels.h"

using namespace tsp;

namespace {

constexpr int64_t MLP_TOKEN_BLOCK = 16384;  // tokens per GELU(x W1^T) workspace block
constexpr size_t WS_ALIGN = 256;

size_t round_up(size_t x) { return (x + WS_ALIGN - 1) / WS_ALIGN * WS_ALIGN; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

tsp_status check_ptr(const void* p) {
  if (!p) return TSP_ERR_INVALID_ARG;
  if (!aligned16(p)) return TSP_ERR_ALIGNMENT;
  return TSP_OK;
}

tsp_status check_ptr_nullable(const void* p) { return (p && !aligned16(p)) ? TSP_ERR_ALIGNMENT : TSP_OK; }

tsp_status check_arrival(const tsp_arrival* a) {
  if (!a || !a->counter || !a->status) return TSP_ERR_INVALID_ARG;
  if (((uintptr_t)a->counter & 3u) || ((uintptr_t)a->status & 3u)) return TSP_ERR_ALIGNMENT;
  return TSP_OK;
}

// The GEMM's shard-arrival fields (nothing when a is null).
void set_arrival(GemmArgs& g, const tsp_arrival* a) {
  if (!a) return;
  g.arrived = a->counter;
  g.arrived_base = a->base;
  g.spin_limit = a->spin_limit ? a->spin_limit : TSP_ARRIVAL_SPIN_DEFAULT;
  g.arrival_status = a->status;
}

// A workspace of `need` bytes: null, misaligned or short is an error unless
// nothing is needed (then the pointer is not used and may be null).
tsp_status check_ws(const void* ws, size_t bytes, size_t need) {
  if (need == 0) return TSP_OK;
  if (!ws) return TSP_ERR_WORKSPACE;
  if (!aligned16(ws)) return TSP_ERR_ALIGNMENT;
  return bytes < need ? TSP_ERR_WORKSPACE : TSP_OK;
}

tsp_status check_shards(const uint16_t* const* w, int32_t D) {
  if (!w) return TSP_ERR_INVALID_ARG;
  for (int d = 0; d < D; ++d) {
    tsp_status s = check_ptr(w[d]);
    if (s != TSP_OK) return s;
  }
  return TSP_OK;
}

// Shape rules shared by every call.  `need_attn` / `need_mlp` add the widths
// the attention and MLP kernels need; `head_shards` (default: need_attn) adds
// that the heads split evenly over the D weight shards, which the attention
// core alone does not need.
tsp_status check_dims(const tsp_dims* d, int32_t D, bool need_attn, bool need_mlp, int head_shards = -1) {
  if (!d) return TSP_ERR_INVALID_ARG;
  if (D < 1 || D > TSP_MAX_D) return TSP_ERR_INVALID_ARG;
  if (d->hidden <= 0 || d->n_heads <= 0 || d->head_dim <= 0 || d->ffn <= 0) return TSP_ERR_SHAPE;
  if ((int64_t)d->n_heads * d->head_dim != d->hidden) return TSP_ERR_SHAPE;
  if (d->hidden % 64 != 0) return TSP_ERR_UNSUPPORTED;
  if (head_shards < 0) head_shards = need_attn ? 1 : 0;
  if (head_shards && d->n_heads % D != 0) return TSP_ERR_SHAPE;
  if (need_attn) {
    if (d->head_dim != 64 && d->head_dim != 128) return TSP_ERR_UNSUPPORTED;
  }
  if (need_mlp) {
    if (d->ffn % D != 0) return TSP_ERR_SHAPE;
    if ((d->ffn / D) % 64 != 0) return TSP_ERR_UNSUPPORTED;
  }
  return TSP_OK;
}

// A plan must be exactly what tsp_zigzag_plan produces for its (S, D, rank).
tsp_status check_plan(const tsp_plan* p) {
  if (!p) return TSP_ERR_INVALID_ARG;
  tsp_plan ref;
  tsp_status s = tsp_zigzag_plan(p->seq_len, p->D, p->rank, &ref, nullptr, nullptr);
  if (s != TSP_OK) return s;
  if (memcmp(&ref, p, sizeof(ref)) != 0) {
    // compare field by field (padding bytes of the caller's struct may differ)
    if (ref.seq_len != p->seq_len || ref.chunk_len != p->chunk_len || ref.n_local != p->n_local ||
        ref.D != p->D || ref.rank != p->rank || ref.chunk_id[0] != p->chunk_id[0] ||
        ref.chunk_id[1] != p->chunk_id[1] || ref.chunk_start[0] != p->chunk_start[0] ||
        ref.chunk_start[1] != p->chunk_start[1])
      return TSP_ERR_SHAPE;
  }
  return TSP_OK;
}

// Attention core workspace: for short sequences, the partial outputs of the
// late chunk's key halves (none otherwise).
size_t ws_core(int64_t n, const tsp_dims* d, int32_t D) {
  return round_up(attn_core_workspace(n * D, n / 2, d->hidden, d->n_heads));
}

// Attention workspace: Q, the attention output as a bf16 pair (hi, lo), then
// the core's split partials.
size_t ws_attn(int64_t n, const tsp_dims* d, int32_t D) {
  return 3 * round_up((size_t)n * d->hidden * 2) + ws_core(n, d, D);
}

// MLP workspace: fp16 GELU output for one token block, the fp16 copy of all W2
// shards, and one int32 row exponent per token.
struct MlpWs {
  size_t h_off, w2_off, exp_off, total;
};

MlpWs mlp_ws(int64_t n, const tsp_dims* d) {
  const int64_t mb = n < MLP_TOKEN_BLOCK ? n : MLP_TOKEN_BLOCK;
  MlpWs w;
  w.h_off = 0;
  w.w2_off = round_up((size_t)mb * d->ffn * 2);
  w.exp_off = w.w2_off + round_up((size_t)d->hidden * d->ffn * 2);
  w.total = w.exp_off + round_up((size_t)n * 4);
  return w;
}

size_t ws_mlp(int64_t n, const tsp_dims* d) { return mlp_ws(n, d).total; }

tsp_status from_hip(hipError_t e) { return e == hipSuccess ? TSP_OK : TSP_ERR_HIP; }

// ---- launches (arguments already validated) ---------------------------------

// QKV projection over all D shards; with an arrival counter, shard d is read
// once ring position (d - start) mod D has arrived.
tsp_status run_project(const tsp_plan* plan, const tsp_dims* dims, const uint16_t* x,
                       const uint16_t* const* wqkv, uint16_t* k_full, uint16_t* v_full, uint16_t* q_out,
                       hipStream_t stream, int32_t start = 0, const tsp_arrival* arr = nullptr) {
  GemmArgs g{};
  g.A = x;
  g.lda = dims->hidden;
  for (int d = 0; d < plan->D; ++d) g.B[d] = wqkv[d];
  const int hs = dims->n_heads / plan->D;
  g.M = (int32_t)plan->n_local;
  g.N_s = 3 * hs * dims->head_dim;
  g.K_s = dims->hidden;
  g.n_shards = plan->D;
  g.k_shards = 1;
  g.ring_start = start;
  set_arrival(g, arr);
  g.epilogue = EPI_QKV;
  g.q_out = q_out;
  g.k_full = k_full;
  g.v_full = v_full;
  g.heads_per_shard = hs;
  g.head_dim = dims->head_dim;
  g.hidden = dims->hidden;
  g.chunk_len = plan->chunk_len;
  g.chunk_start0 = plan->chunk_start[0];
  g.chunk_start1 = plan->chunk_start[1];
  return from_hip(launch_gemm(g, stream));
}

tsp_status run_core(const tsp_plan* plan, const tsp_dims* dims, const uint16_t* q, const uint16_t* k_full,
                    const uint16_t* v_full, uint16_t* attn_out, uint16_t* attn_lo, void* core_ws,
                    hipStream_t stream, float* lse = nullptr) {
  AttnArgs a{};
  a.lse = lse;
  a.q = q;
  a.k = k_full;
  a.v = v_full;
  a.o = attn_out;
  a.o_lo = attn_lo;
  a.seq_len = plan->seq_len;
  a.chunk_len = plan->chunk_len;
  a.chunk_start0 = plan->chunk_start[0];
  a.chunk_start1 = plan->chunk_start[1];
  a.hidden = dims->hidden;
  a.n_heads = dims->n_heads;
  a.head_dim = dims->head_dim;
  a.kv_heads = dims->n_heads;
  a.kv_ld = dims->hidden;
  a.ws = core_ws;
  return from_hip(launch_attention(a, stream));
}

tsp_status run_out(int64_t n, const tsp_dims* dims, int32_t D, int32_t start, const uint16_t* attn,
                   const uint16_t* attn_lo, const uint16_t* const* wo, const uint16_t* residual, void* out,
                   bool out_f32, hipStream_t stream, const tsp_arrival* arr = nullptr) {
  GemmArgs g{};
  set_arrival(g, arr);
  g.A = attn;
  g.A_lo = attn_lo;
  g.lda = dims->hidden;
  for (int d = 0; d < D; ++d) g.B[d] = wo[d];
  g.M = (int32_t)n;
  g.N_s = dims->hidden;
  g.K_s = (dims->n_heads / D) * dims->head_dim;
  g.n_shards = 1;
  g.k_shards = D;
  g.ring_start = start;
  g.epilogue = EPI_RESID;
  g.out = out;
  g.out_f32 = out_f32;
  g.ldo = dims->hidden;
  g.residual = residual;
  return from_hip(launch_gemm(g, stream));
}

// The two MLP GEMMs over token blocks.  `a` holds the MLP input rows: bf16, or
// (a_f16) fp16 scaled by 2^-row_exp.  `w1` are bf16 or fp16 shards to match;
// `w2h` is the fp16 copy of the W2 shards (D blocks of [hidden x F_s]).
// y = [residual +] sum_k GELU(x W1_{d_k}^T) W2_{d_k}^T, fp32 across all shards.
// With an arrival counter the W1 GEMMs wait for their shards; `after_w1`
// (nullable) runs after the first token block's W1 GEMM, which has then seen
// every shard pair arrive.
tsp_status run_mlp_core(int64_t n, const tsp_dims* dims, int32_t D, int32_t start, const uint16_t* a, bool a_f16,
                        const uint16_t* const* w1, const uint16_t* w2h, const int32_t* row_exp,
                        const void* residual, bool res_f32, uint16_t* y, uint16_t* hbuf, hipStream_t stream,
                        const tsp_arrival* arr = nullptr, const std::function<tsp_status()>& after_w1 = {}) {
  const int64_t h = dims->hidden;
  const int32_t fs = dims->ffn / D;
  for (int64_t b0 = 0; b0 < n; b0 += MLP_TOKEN_BLOCK) {
    const int64_t mb = (n - b0) < MLP_TOKEN_BLOCK ? (n - b0) : MLP_TOKEN_BLOCK;
    // fp16(GELU(x W1_d^T) * 2^-row_exp) for every shard d -> hbuf[:, d*F_s .. (d+1)*F_s)
    GemmArgs g1{};
    g1.f16 = a_f16;
    g1.A = a + b0 * h;
    g1.lda = h;
    for (int d = 0; d < D; ++d) g1.B[d] = w1[d];
    g1.M = (int32_t)mb;
    g1.N_s = fs;
    g1.K_s = (int32_t)h;
    g1.n_shards = D;
    g1.k_shards = 1;
    g1.epilogue = EPI_GELU;
    g1.out = hbuf;
    g1.ldo = dims->ffn;
    g1.row_exp = row_exp + b0;
    g1.gelu_in_scaled = a_f16;
    g1.ring_start = start;
    set_arrival(g1, arr);
    tsp_status s = from_hip(launch_gemm(g1, stream));
    if (s != TSP_OK) return s;
    if (b0 == 0 && after_w1 && (s = after_w1()) != TSP_OK) return s;
    // y = [residual +] 2^row_exp * sum over shards in ring order of hbuf[:, d block] W2_d^T
    GemmArgs g2{};
    g2.f16 = 1;
    g2.A = hbuf;
    g2.lda = dims->ffn;
    for (int d = 0; d < D; ++d) g2.B[d] = w2h + (int64_t)d * h * fs;
    g2.M = (int32_t)mb;
    g2.N_s = (int32_t)h;
    g2.K_s = fs;
    g2.n_shards = 1;
    g2.k_shards = D;
    g2.ring_start = start;
    g2.epilogue = EPI_RESID;
    g2.out = y + b0 * h;
    g2.ldo = h;
    if (residual)
      g2.residual = res_f32 ? (const void*)(static_cast<const float*>(residual) + b0 * h)
                            : (const void*)(static_cast<const uint16_t*>(residual) + b0 * h);
    g2.res_f32 = res_f32;
    g2.row_exp = row_exp + b0;
    s = from_hip(launch_gemm(g2, stream));
    if (s != TSP_OK) return s;
  }
  return TSP_OK;
}

tsp_status run_mlp(int64_t n, const tsp_dims* dims, int32_t D, int32_t start, const uint16_t* x,
                   const uint16_t* const* w1, const uint16_t* const* w2, const uint16_t* residual, uint16_t* y,
                   void* ws, hipStream_t stream, const tsp_arrival* arr = nullptr) {
  if (n == 0) return TSP_OK;
  const MlpWs lay = mlp_ws(n, dims);
  char* base = static_cast<char*>(ws);
  uint16_t* hbuf = reinterpret_cast<uint16_t*>(base + lay.h_off);
  uint16_t* w2h = reinterpret_cast<uint16_t*>(base + lay.w2_off);
  int32_t* row_exp = reinterpret_cast<int32_t*>(base + lay.exp_off);
  tsp_status s = from_hip(launch_row_prep(x, 0, n, dims->hidden, row_exp, nullptr, stream));
  if (s != TSP_OK) return s;
  auto convert_w2 = [&]() { return from_hip(launch_bf16_to_f16(w2, w2h, D, (int64_t)dims->hidden * (dims->ffn / D), stream)); };
  if (!arr) {  // the copy first: the W1 and W2 GEMMs of each token block then run back to back
    if ((s = convert_w2()) != TSP_OK) return s;
    return run_mlp_core(n, dims, D, start, x, false, w1, w2h, row_exp, residual, false, y, hbuf, stream);
  }
  return run_mlp_core(n, dims, D, start, x, false, w1, w2h, row_exp, residual, false, y, hbuf, stream, arr,
                      convert_w2);
}

// Workspace of the post-attention half of the layer: fp32 h1, its scaled fp16
// copy, row exponents, fp16 W1 and W2 shards and the fp16 GELU block.
struct PostWs {
  size_t h1_off, h16_off, exp_off, w1_off, w2_off, hbuf_off, total;
};

PostWs post_ws(int64_t n, const tsp_dims* d) {
  const int64_t mb = n < MLP_TOKEN_BLOCK ? n : MLP_TOKEN_BLOCK;
  PostWs w;
  w.h1_off = 0;
  w.h16_off = round_up((size_t)n * d->hidden * 4);
  w.exp_off = w.h16_off + round_up((size_t)n * d->hidden * 2);
  w.w1_off = w.exp_off + round_up((size_t)n * 4);
  w.w2_off = w.w1_off + round_up((size_t)d->ffn * d->hidden * 2);
  w.hbuf_off = w.w2_off + round_up((size_t)d->ffn * d->hidden * 2);
  w.total = w.hbuf_off + round_up((size_t)mb * d->ffn * 2);
  return w;
}

// Whole layer: Q and attention-output buffers, then the post workspace.
size_t ws_layer(int64_t n, const tsp_dims* d, int32_t D) { return ws_attn(n, d, D) + post_ws(n, d).total; }

// h1 = x + attn W_o^T (fp32, split-K over head shards from `start`), then
// out = h1 + MLP(h1) on scaled fp16 operands with the ring from `start`.
tsp_status run_post(int64_t n, const tsp_dims* dims, int32_t D, int32_t start, const uint16_t* attn,
                    const uint16_t* attn_lo, const uint16_t* x, const uint16_t* const* wo, const uint16_t* const* w1,
                    const uint16_t* const* w2, uint16_t* out, void* ws, hipStream_t stream) {
  if (n == 0) return TSP_OK;
  const PostWs lay = post_ws(n, dims);
  char* base = static_cast<char*>(ws);
  float* h1 = reinterpret_cast<float*>(base + lay.h1_off);
  uint16_t* h16 = reinterpret_cast<uint16_t*>(base + lay.h16_off);
  int32_t* row_exp = reinterpret_cast<int32_t*>(base + lay.exp_off);
  uint16_t* w1h = reinterpret_cast<uint16_t*>(base + lay.w1_off);
  uint16_t* w2h = reinterpret_cast<uint16_t*>(base + lay.w2_off);
  uint16_t* hbuf = reinterpret_cast<uint16_t*>(base + lay.hbuf_off);
  const int64_t shard_elems = (int64_t)dims->hidden * (dims->ffn / D);
  tsp_status s;
  if ((s = run_out(n, dims, D, start, attn, attn_lo, wo, x, h1, true, stream)) != TSP_OK) return s;
  if ((s = from_hip(launch_row_prep(h1, 1, n, dims->hidden, row_exp, h16, stream))) != TSP_OK) return s;
  if ((s = from_hip(launch_bf16_to_f16(w1, w1h, D, shard_elems, stream))) != TSP_OK) return s;
  if ((s = from_hip(launch_bf16_to_f16(w2, w2h, D, shard_elems, stream))) != TSP_OK) return s;
  const uint16_t* w1h_shards[TSP_MAX_D];
  for (int d = 0; d < D; ++d) w1h_shards[d] = w1h + d * shard_elems;
  return run_mlp_core(n, dims, D, start, h16, true, w1h_shards, w2h, row_exp, h1, true, out, hbuf, stream);
}

// Shapes of grouped-query attention: query heads in groups over the K/V heads.
tsp_status check_gqa(const tsp_dims* dims, int32_t D, int32_t n_kv_heads, bool sharded) {
  if (n_kv_heads <= 0 || n_kv_heads > dims->n_heads || dims->n_heads % n_kv_heads != 0) return TSP_ERR_SHAPE;
  if (sharded && n_kv_heads % D != 0) return TSP_ERR_SHAPE;
  return TSP_OK;
}

// ---- MLP backward --------------------------------------------------------------

// Workspace of tsp_mlp_backward (n_pad = n rounded up to 64): x^T and dy^T
// [h x n_pad], U_d fp32 [n x F_s], GELU(U)^T and dU^T of all shards
// [F x n_pad], dU of all shards [n x F], W1_d^T of all shards [D][h x F_s],
// W2_d^T [F_s x h].
struct MlpBwdWs {
  size_t xt_off, dyt_off, u_off, ht_off, dut_off, du_off, w1t_off, w2t_off, total;
};

int64_t pad64(int64_t n) { return (n + 63) / 64 * 64; }

MlpBwdWs mlp_bwd_ws(int64_t n, const tsp_dims* d, int32_t D) {
  const int64_t np = pad64(n), h = d->hidden, F = d->ffn, fs = F / D;
  MlpBwdWs w;
  w.xt_off = 0;
  w.dyt_off = w.xt_off + round_up((size_t)h * np * 2);
  w.u_off = w.dyt_off + round_up((size_t)h * np * 2);
  w.ht_off = w.u_off + round_up((size_t)n * fs * 4);
  w.dut_off = w.ht_off + round_up((size_t)F * np * 2);
  w.du_off = w.dut_off + round_up((size_t)F * np * 2);
  w.w1t_off = w.du_off + round_up((size_t)n * F * 2);
  w.w2t_off = w.w1t_off + round_up((size_t)h * F * 2);
  w.total = w.w2t_off + round_up((size_t)fs * h * 2);
  return w;
}

// Workspace of tsp_attn_out_backward: W_o_d^T of all shards [D][H_s*hd x h],
// d_out^T [h x n_pad], attn^T [h x n_pad].
struct OutBwdWs {
  size_t wot_off, dot_off, at_off, total;
};
OutBwdWs out_bwd_ws(int64_t n, const tsp_dims* d, int32_t D) {
  const int64_t np = pad64(n), h = d->hidden, hs = (int64_t)(d->n_heads / D) * d->head_dim;
  OutBwdWs w;
  w.wot_off = 0;
  w.dot_off = w.wot_off + round_up((size_t)h * h * 2);
  w.at_off = w.dot_off + round_up((size_t)h * np * 2);
  w.total = w.at_off + round_up((size_t)h * np * 2);
  return w;
}

// Workspace of tsp_attn_project_backward: G = bf16[dq | dk | dv] [n x 3h], x^T
// [h x n_pad], [dq_d | dk_d | dv_d]^T of all shards [D][3 H_s*hd x n_pad], and
// the transposed Q, K and V weight blocks of all shards [3][D][h x H_s*hd].
struct ProjBwdWs {
  size_t g_off, xt_off, gt_off, wt_off, total;
};
ProjBwdWs proj_bwd_ws(int64_t n, const tsp_dims* d, int32_t D) {
  const int64_t np = pad64(n), h = d->hidden, hs = (int64_t)(d->n_heads / D) * d->head_dim;
  ProjBwdWs w;
  w.g_off = 0;
  w.xt_off = w.g_off + round_up((size_t)n * 3 * h * 2);
  w.gt_off = w.xt_off + round_up((size_t)h * np * 2);
  w.wt_off = w.gt_off + round_up((size_t)3 * h * np * 2);
  w.total = w.wt_off + round_up((size_t)3 * h * h * 2);
  return w;
}

// ---- shard streaming ---------------------------------------------------------

// O projection ring step: the fp32 accumulator [n x h].
size_t ws_out_shard(int64_t n, const tsp_dims* d) { return round_up((size_t)n * d->hidden * 4); }

// MLP ring step: fp32 accumulator, row exponents, the fp16 copy of W2_d and the
// fp16 GELU block of the shard (F_s columns).
struct MlpShardWs {
  size_t acc_off, exp_off, w2_off, h_off, total;
};

MlpShardWs mlp_shard_ws(int64_t n, const tsp_dims* d, int32_t D) {
  const int64_t mb = n < MLP_TOKEN_BLOCK ? n : MLP_TOKEN_BLOCK;
  const int64_t fs = d->ffn / D;
  MlpShardWs w;
  w.acc_off = 0;
  w.exp_off = round_up((size_t)n * d->hidden * 4);
  w.w2_off = w.exp_off + round_up((size_t)n * 4);
  w.h_off = w.w2_off + round_up((size_t)d->hidden * fs * 2);
  w.total = w.h_off + round_up((size_t)mb * fs * 2);
  return w;
}

// Residual and output of ring step pos of D: the caller's residual (bf16,
// nullable) at the first step, else the fp32 accumulator; the caller's bf16
// output at the last step, else the accumulator.
void ring_io(GemmArgs& g, int32_t D, int32_t pos, const uint16_t* residual, uint16_t* out, float* acc,
             int64_t row0, int64_t ld) {
  if (pos == 0) {
    g.residual = residual ? (const void*)(residual + row0 * ld) : nullptr;
    g.res_f32 = 0;
  } else {
    g.residual = acc + row0 * ld;
    g.res_f32 = 1;
  }
  if (pos == D - 1) {
    g.out = out + row0 * ld;
    g.out_f32 = 0;
  } else {
    g.out = acc + row0 * ld;
    g.out_f32 = 1;
  }
}

tsp_status run_attn_backward(const tsp_plan* plan, const tsp_dims* dims, int32_t kv_heads, const uint16_t* q,
                             const uint16_t* k_full, const uint16_t* v_full, const uint16_t* attn_out,
                             const uint16_t* attn_lo, const float* lse, const uint16_t* d_attn, float* dq,
                             float* dk_full, float* dv_full, void* workspace, size_t ws_bytes, hipStream_t stream) {
  tsp_status s;
  if ((s = check_ptr(q)) != TSP_OK || (s = check_ptr(k_full)) != TSP_OK || (s = check_ptr(v_full)) != TSP_OK ||
      (s = check_ptr(attn_out)) != TSP_OK || (s = check_ptr_nullable(attn_lo)) != TSP_OK ||
      (s = check_ptr(lse)) != TSP_OK || (s = check_ptr(d_attn)) != TSP_OK || (s = check_ptr(dq)) != TSP_OK ||
      (s = check_ptr(dk_full)) != TSP_OK || (s = check_ptr(dv_full)) != TSP_OK)
    return s;
  if (dk_full == dv_full || (void*)dq == (void*)dk_full || (void*)dq == (void*)dv_full) return TSP_ERR_INVALID_ARG;
  const size_t need = attn_bwd_ws_bytes(plan->seq_len, plan->chunk_len, dims->n_heads, kv_heads, dims->head_dim);
  if (!workspace) return TSP_ERR_WORKSPACE;
  if (!aligned16(workspace)) return TSP_ERR_ALIGNMENT;
  if (ws_bytes < need) return TSP_ERR_WORKSPACE;
  AttnBwdArgs a{};
  a.q = q;
  a.k = k_full;
  a.v = v_full;
  a.o = attn_out;
  a.o_lo = attn_lo;
  a.dout = d_attn;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk_full;
  a.dv = dv_full;
  a.seq_len = plan->seq_len;
  a.chunk_len = plan->chunk_len;
  a.chunk_start0 = plan->chunk_start[0];
  a.chunk_start1 = plan->chunk_start[1];
  a.hidden = dims->hidden;
  a.n_heads = dims->n_heads;
  a.head_dim = dims->head_dim;
  a.kv_heads = kv_heads;
  a.kv_ld = kv_heads * dims->head_dim;
  a.n_kv_tiles = (plan->seq_len + 63) / 64;
  a.tpc = (plan->chunk_len + 63) / 64;
  // workspace: K^T tiles, Q^T tiles, dO^T tiles (these three at head_dim 64
  // only), stats (each size a multiple of 1 KB)
  uint8_t* w = static_cast<uint8_t*>(workspace);
  if (attn_bwd_stages_kt(dims->head_dim)) {
    a.kt = reinterpret_cast<uint16_t*>(w);
    w += (size_t)kv_heads * a.n_kv_tiles * dims->head_dim * 64 * 2;
  }
  if (attn_bwd_stages_qt(dims->head_dim)) {
    a.qt = reinterpret_cast<uint16_t*>(w);
    w += (size_t)2 * dims->n_heads * a.tpc * dims->head_dim * 64 * 2;
    a.dot = reinterpret_cast<uint16_t*>(w);
    w += (size_t)2 * dims->n_heads * a.tpc * dims->head_dim * 64 * 2;
  }
  a.stats = reinterpret_cast<float*>(w);
  return from_hip(launch_attention_backward(a, stream));
}

}  // namespace

extern "C" {

tsp_status tsp_zigzag_plan(int64_t seq_len, int32_t D, int32_t rank, tsp_plan* plan, int64_t* local_to_global,
                           int32_t* ring_order) {
  if (!plan) return TSP_ERR_INVALID_ARG;
  if (D < 1 || D > TSP_MAX_D) return TSP_ERR_INVALID_ARG;
  if (rank < 0 || rank >= D) return TSP_ERR_INVALID_ARG;
  if (seq_len <= 0 || seq_len % (2 * (int64_t)D) != 0) return TSP_ERR_SHAPE;
  if (seq_len / D > INT32_MAX) return TSP_ERR_UNSUPPORTED;
  tsp_plan p;
  memset(&p, 0, sizeof(p));
  p.seq_len = seq_len;
  p.D = D;
  p.rank = rank;
  p.chunk_len = seq_len / (2 * (int64_t)D);
  p.n_local = 2 * p.chunk_len;
  p.chunk_id[0] = rank;
  p.chunk_id[1] = 2 * D - 1 - rank;
  p.chunk_start[0] = (int64_t)p.chunk_id[0] * p.chunk_len;
  p.chunk_start[1] = (int64_t)p.chunk_id[1] * p.chunk_len;
  if (local_to_global) {
    for (int64_t i = 0; i < p.n_local; ++i)
      local_to_global[i] = i < p.chunk_len ? p.chunk_start[0] + i : p.chunk_start[1] + (i - p.chunk_len);
  }
  if (ring_order) {
    for (int k = 0; k < D; ++k) ring_order[k] = (rank + k) % D;
  }
  *plan = p;
  return TSP_OK;
}

size_t tsp_workspace_size(int64_t n_tokens, const tsp_dims* dims, int32_t D, int32_t kind) {
  if (n_tokens < 0) return 0;
  switch (kind) {
    case TSP_WS_ATTN:
      if (check_dims(dims, D, true, false) != TSP_OK) return 0;
      return ws_attn(n_tokens, dims, D);
    case TSP_WS_CORE:
      if (check_dims(dims, D, true, false, 0) != TSP_OK) return 0;
      return ws_core(n_tokens, dims, D);
    case TSP_WS_MLP:
      if (check_dims(dims, D, false, true) != TSP_OK) return 0;
      return ws_mlp(n_tokens, dims);
    case TSP_WS_LAYER:
      if (check_dims(dims, D, true, true) != TSP_OK) return 0;
      return ws_layer(n_tokens, dims, D);
    case TSP_WS_POST:
      if (check_dims(dims, D, true, true) != TSP_OK) return 0;
      return post_ws(n_tokens, dims).total;
    case TSP_WS_OUT_SHARD:
      if (check_dims(dims, D, true, false) != TSP_OK) return 0;
      return ws_out_shard(n_tokens, dims);
    case TSP_WS_MLP_SHARD:
      if (check_dims(dims, D, false, true) != TSP_OK) return 0;
      return mlp_shard_ws(n_tokens, dims, D).total;
    case TSP_WS_MLP_BWD:
      if (check_dims(dims, D, false, true) != TSP_OK) return 0;
      return mlp_bwd_ws(n_tokens, dims, D).total;
    case TSP_WS_OUT_BWD:
      if (check_dims(dims, D, true, false) != TSP_OK) return 0;
      return out_bwd_ws(n_tokens, dims, D).total;
    case TSP_WS_PROJ_BWD:
      if (check_dims(dims, D, true, false) != TSP_OK) return 0;
      return proj_bwd_ws(n_tokens, dims, D).total;
    case TSP_WS_RMS_BWD:
      if (!dims || dims->hidden <= 0) return 0;
      return round_up((size_t)rms_norm_bwd_blocks(n_tokens) * dims->hidden * 4);
    case TSP_WS_ATTN_BWD:
      if (check_dims(dims, D, true, false, 0) != TSP_OK || n_tokens % 2 != 0) return 0;
      return attn_bwd_ws_bytes(n_tokens * D, n_tokens / 2, dims->n_heads, dims->n_heads, dims->head_dim);
    default:
      return 0;
  }
}

tsp_status tsp_attn_project(const tsp_plan* plan, const tsp_dims* dims, const uint16_t* x_local,
                            const uint16_t* const* wqkv, uint16_t* k_full, uint16_t* v_full, uint16_t* q_out,
                            hipStream_t stream) {
  tsp_status s;
  if ((s = check_plan(plan)) != TSP_OK) return s;
  if ((s = check_dims(dims, plan->D, true, false)) != TSP_OK) return s;
  if ((s = check_ptr(x_local)) != TSP_OK || (s = check_shards(wqkv, plan->D)) != TSP_OK ||
      (s = check_ptr(k_full)) != TSP_OK || (s = check_ptr(v_full)) != TSP_OK || (s = check_ptr(q_out)) != TSP_OK)
    return s;
  return run_project(plan, dims, x_local, wqkv, k_full, v_full, q_out, stream);
}

tsp_status tsp_attn_core(const tsp_plan* plan, const tsp_dims* dims, const uint16_t* q, const uint16_t* k_full,
                         const uint16_t* v_full, uint16_t* attn_out, uint16_t* attn_lo, void* workspace,
                         size_t ws_bytes, hipStream_t stream) {
  tsp_status s;
  if ((s = check_plan(plan)) != TSP_OK) return s;
  if ((s = check_dims(dims, plan->D, true, false, 0)) != TSP_OK) return s;
  if ((s = check_ptr(q)) != TSP_OK || (s = check_ptr(k_full)) != TSP_OK || (s = check_ptr(v_full)) != TSP_OK ||
      (s = check_ptr(attn_out)) != TSP_OK || (s = check_ptr_nullable(attn_lo)) != TSP_OK)
    return s;
  if (attn_out == q || attn_lo == q || attn_lo == attn_out) return TSP_ERR_INVALID_ARG;
  if ((s = check_ws(workspace, ws_bytes, ws_core(plan->n_local, dims, plan->D))) != TSP_OK) return s;
  return run_core(plan, dims, q, k_full, v_full, attn_out, attn_lo, workspace, stream);
}

tsp_status tsp_attn_core_lse(const tsp_plan* plan, const tsp_dims* dims, const uint16_t* q, const uint16_t* k_full,
                             const uint16_t* v_full, uint16_t* attn_out, uint16_t* attn_lo, float* lse,
                             void* workspace, size_t ws_bytes, hipStream_t stream) {
  tsp_status s;
  if ((s = check_plan(plan)) != TSP_OK) return s;
  if ((s = check_dims(dims, plan->D, true, false, 0)) != TSP_OK) return s;
  if ((s = check_ptr(q)) != TSP_OK || (s = check_ptr(k_full)) != TSP_OK || (s = check_ptr(v_full)) != TSP_OK ||
      (s = check_ptr(attn_out)) != TSP_OK || (s = check_ptr_nullable(attn_lo)) != TSP_OK ||
      (s = check_ptr(lse)) != TSP_OK)
    return s;
  if (attn_out == q || attn_lo == q || attn_lo == attn_out) return TSP_ERR_INVALID_ARG;
  if ((s = check_ws(workspace, ws_bytes, ws_core(plan->n_local, dims, plan->D))) != TSP_OK) return s;
  return run_core(plan, dims, q, k_full, v_full, attn_out, attn_lo, workspace, stream, lse);
}


tsp_status tsp_attn_core_backward(const tsp_plan* plan, const tsp_dims* dims, const uint16_t* q,
                                  const uint16_t* k_full, const uint16_t* v_full, const uint16_t* attn_out,
                                  const uint16_t* attn_lo, const float* lse, const uint16_t* d_attn, float* dq,
                                  float* dk_full, float* dv_full, void* workspace, size_t ws_bytes,
                                  hipStream_t stream) {
  tsp_status s;
  if ((s = check_plan(plan)) != TSP_OK) return s;
  if ((s = check_dims(dims, plan->D, true, false, 0)) != TSP_OK) return s;
  return run_attn_backward(plan, dims, dims->n_heads, q, k_full, v_full, attn_out, attn_lo, lse, d_attn, dq,
                           dk_full, dv_full, workspace, ws_bytes, stream);
}

tsp_status tsp_attn_out(int64_t n_tokens, const tsp_dims* dims, int32_t D, int32_t start_shard,
                        const uint16_t* attn, const uint16_t* attn_lo, const uint16_t* const* wo,
                        const uint16_t* residual, uint16_t* out, hipStream_t stream) {
  tsp_status s;
  if ((s = check_dims(dims, D, true, false)) != TSP_OK) return s;
  if (n_tokens < 0) return TSP_ERR_SHAPE;
  if (n_tokens > INT32_MAX) return TSP_ERR_UNSUPPORTED;
  if (start_shard < 0 || start_shard >= D) return TSP_ERR_INVALID_ARG;
  if ((s = check_ptr(attn)) != TSP_OK || (s = check_ptr_nullable(attn_lo)) != TSP_OK ||
      (s = check_shards(wo, D)) != TSP_OK || (s = check_ptr_nullable(residual)) != TSP_OK ||
      (s = check_ptr(out)) != TSP_OK)
    return s;
  if (out == attn || (attn_lo && out == attn_lo)) return TSP_ERR_INVALID_ARG;
  return run_out(n_tokens, dims, D, start_shard, attn, attn_lo, wo, residual, out, false, stream);
}

tsp_status tsp_attn_forward(const tsp_plan* plan, const tsp_dims* dims, const uint16_t* x_local,
                            const uint16_t* const* wqkv, const uint16_t* const* wo, uint16_t* k_full,
                            uint16_t* v_full, const uint16_t* residual, uint16_t* out, void* workspace,
                            size_t ws_bytes, hipStream_t stream) {
  tsp_status s;
  if ((s = check_plan(plan)) != TSP_OK) return s;
  if ((s = check_dims(dims, plan->D, true, false)) != TSP_OK) return s;
  if ((s = check_ptr(x_local)) != TSP_OK || (s = check_shards(wqkv, plan->D)) != TSP_OK ||
      (s = check_shards(wo, plan->D)) != TSP_OK || (s = check_ptr(k_full)) != TSP_OK ||
      (s = check_ptr(v_full)) != TSP_OK || (s = check_ptr_nullable(residual)) != TSP_OK ||
      (s = check_ptr(out)) != TSP_OK)
    return s;
  if (out == x_local) return TSP_ERR_INVALID_ARG;
  if (!workspace) return TSP_ERR_WORKSPACE;
  if (!aligned16(workspace)) return TSP_ERR_ALIGNMENT;
  if (ws_bytes < ws_attn(plan->n_local, dims, plan->D)) return TSP_ERR_WORKSPACE;
  uint16_t* qbuf = static_cast<uint16_t*>(workspace);
  uint16_t* abuf = qbuf + round_up((size_t)plan->n_local * dims->hidden * 2) / 2;
  uint16_t* alo = abuf + round_up((size_t)plan->n_local * dims->hidden * 2) / 2;
  void* core_ws = alo + round_up((size_t)plan->n_local * dims->hidden * 2) / 2;
  if ((s = run_project(plan, dims, x_local, wqkv, k_full, v_full, qbuf, stream)) != TSP_OK) return s;
  if ((s = run_core(plan, dims, qbuf, k_full, v_full, abuf, alo, core_ws, stream)) != TSP_OK) return s;
  return run_out(plan->n_local, dims, plan->D, plan->rank, abuf, alo, wo, residual, out, false, stream);
}

tsp_status tsp_mlp_forward(int64_t n_tokens, const tsp_dims* dims, int32_t D, int32_t start_shard,
                           const uint16_t* x, const uint16_t* const* w1, const uint16_t* const* w2,
                           const uint16_t* residual, uint16_t* y, void* workspace, size_t ws_bytes,
                           hipStream_t stream) {
  tsp_status s;
  if ((s = check_dims(dims, D, false, true)) != TSP_OK) return s;
  if (n_tokens < 0) return TSP_ERR_SHAPE;
  if (n_tokens > INT32_MAX) return TSP_ERR_UNSUPPORTED;
  if (start_shard < 0 || start_shard >= D) return TSP_ERR_INVALID_ARG;
  if ((s = check_ptr(x)) != TSP_OK || (s = check_shards(w1, D)) != TSP_OK || (s = check_shards(w2, D)) != TSP_OK ||
      (s = check_ptr_nullable(residual)) != TSP_OK || (s = check_ptr(y)) != TSP_OK)
    return s;
  if (y == x && residual != x) return TSP_ERR_INVALID_ARG;
  if (!workspace) return TSP_ERR_WORKSPACE;
  if (!aligned16(workspace)) return TSP_ERR_ALIGNMENT;
  if (ws_bytes < ws_mlp(n_tokens, dims)) return TSP_ERR_WORKSPACE;
  return run_mlp(n_tokens, dims, D, start_shard, x, w1, w2, residual, y, workspace, stream);
}

tsp_status tsp_layer_forward(const tsp_plan* plan, const tsp_dims* dims, const uint16_t* x_local,
                             const uint16_t* const* wqkv, const uint16_t* const* wo, const uint16_t* const* w1,
                             const uint16_t* const* w2, uint16_t* k_full, uint16_t* v_full, uint16_t* out,
                             void* workspace, size_t ws_bytes, hipStream_t stream) {
  tsp_status s;
  if ((s = check_plan(plan)) != TSP_OK) return s;
  if ((s = check_dims(dims, plan->D, true, true)) != TSP_OK) return s;
  if ((s = check_ptr(x_local)) != TSP_OK || (s = check_shards(wqkv, plan->D)) != TSP_OK ||
      (s = check_shards(wo, plan->D)) != TSP_OK || (s = check_shards(w1, plan->D)) != TSP_OK ||
      (s = check_shards(w2, plan->D)) != TSP_OK || (s = check_ptr(k_full)) != TSP_OK ||
      (s = check_ptr(v_full)) != TSP_OK || (s = check_ptr(out)) != TSP_OK)
    return s;
  if (out == x_local) return TSP_ERR_INVALID_ARG;
  if (!workspace) return TSP_ERR_WORKSPACE;
  if (!aligned16(workspace)) return TSP_ERR_ALIGNMENT;
  const int64_t n = plan->n_local;
  if (ws_bytes < ws_layer(n, dims, plan->D)) return TSP_ERR_WORKSPACE;
  uint16_t* qbuf = static_cast<uint16_t*>(workspace);
  uint16_t* abuf = qbuf + round_up((size_t)n * dims->hidden * 2) / 2;
  uint16_t* alo = abuf + round_up((size_t)n * dims->hidden * 2) / 2;
  void* core_ws = alo + round_up((size_t)n * dims->hidden * 2) / 2;
  char* post = static_cast<char*>(workspace) + ws_attn(n, dims, plan->D);
  if ((s = run_project(plan, dims, x_local, wqkv, k_full, v_full, qbuf, stream)) != TSP_OK) return s;
  if ((s = run_core(plan, dims, qbuf, k_full, v_full, abuf, alo, core_ws, stream)) != TSP_OK) return s;
  return run_post(n, dims, plan->D, plan->rank, abuf, alo, x_local, wo, w1, w2, out, post, stream);
}

tsp_status tsp_layer_post(int64_t n_tokens, const tsp_dims* dims, int32_t D, int32_t start_shard,
                          const uint16_t* attn, const uint16_t* attn_lo, const uint16_t* x,
                          const uint16_t* const* wo, const uint16_t* const* w1, const uint16_t* const* w2,
                          uint16_t* out, void* workspace, size_t ws_bytes, hipStream_t stream) {
  tsp_status s;
  if ((s = check_dims(dims, D, true, true)) != TSP_OK) return s;
  if (n_tokens < 0) return TSP_ERR_SHAPE;
  if (n_tokens > INT32_MAX) return TSP_ERR_UNSUPPORTED;
  if (start_shard < 0 || start_shard >= D) return TSP_ERR_INVALID_ARG;
  if ((s = check_ptr(attn)) != TSP_OK || (s = check_ptr_nullable(attn_lo)) != TSP_OK ||
      (s = check_ptr(x)) != TSP_OK || (s = check_shards(wo, D)) != TSP_OK ||
      (s = check_shards(w1, D)) != TSP_OK || (s = check_shards(w2, D)) != TSP_OK || (s = check_ptr(out)) != TSP_OK)
    return s;
  if (out == x || out == attn || (attn_lo && out == attn_lo)) return TSP_ERR_INVALID_ARG;
  if (!workspace) return TSP_ERR_WORKSPACE;
  if (!aligned16(workspace)) return TSP_ERR_ALIGNMENT;
  if (ws_bytes < post_ws(n_tokens, dims).total) return TSP_ERR_WORKSPACE;
  return run_post(n_tokens, dims, D, start_shard, attn, attn_lo, x, wo, w1, w2, out, workspace, stream);
}

tsp_status tsp_attn_project_shard(const tsp_plan* plan, const tsp_dims* dims, int32_t shard,
                                  const uint16_t* x_local, const uint16_t* wqkv_d, uint16_t* k_full,
                                  uint16_t* v_full, uint16_t* q_out, hipStream_t stream) {
  tsp_status s;
  if ((s = check_plan(plan)) != TSP_OK) return s;
  if ((s = check_dims(dims, plan->D, true, false)) != TSP_OK) return s;
  if (shard < 0 || shard >= plan->D) return TSP_ERR_INVALID_ARG;
  if ((s = check_ptr(x_local)) != TSP_OK || (s = check_ptr(wqkv_d)) != TSP_OK ||
      (s = check_ptr(k_full)) != TSP_OK || (s = check_ptr(v_full)) != TSP_OK || (s = check_ptr(q_out)) != TSP_OK)
    return s;
  GemmArgs g{};
  g.A = x_local;
  g.lda = dims->hidden;
  g.B[0] = wqkv_d;
  const int hs = dims->n_heads / plan->D;
  g.M = (int32_t)plan->n_local;
  g.N_s = 3 * hs * dims->head_dim;
  g.K_s = dims->hidden;
  g.n_shards = 1;
  g.k_shards = 1;
  g.epilogue = EPI_QKV;
  g.q_out = q_out;
  g.k_full = k_full;
  g.v_full = v_full;
  g.heads_per_shard = hs;
  g.head_dim = dims->head_dim;
  g.hidden = dims->hidden;
  g.shard0 = shard;
  g.chunk_len = plan->chunk_len;
  g.chunk_start0 = plan->chunk_start[0];
  g.chunk_start1 = plan->chunk_start[1];
  return from_hip(launch_gemm(g, stream));
}

tsp_status tsp_attn_out_shard(int64_t n_tokens, const tsp_dims* dims, int32_t D, int32_t pos, int32_t shard,
                              const uint16_t* attn, const uint16_t* attn_lo, const uint16_t* wo_d,
                              const uint16_t* residual, uint16_t* out, void* workspace, size_t ws_bytes,
                              hipStream_t stream) {
  tsp_status s;
  if ((s = check_dims(dims, D, true, false)) != TSP_OK) return s;
  if (n_tokens < 0) return TSP_ERR_SHAPE;
  if (n_tokens > INT32_MAX) return TSP_ERR_UNSUPPORTED;
  if (pos < 0 || pos >= D || shard < 0 || shard >= D) return TSP_ERR_INVALID_ARG;
  if ((s = check_ptr(attn)) != TSP_OK || (s = check_ptr_nullable(attn_lo)) != TSP_OK ||
      (s = check_ptr(wo_d)) != TSP_OK || (s = check_ptr_nullable(residual)) != TSP_OK ||
      (s = check_ptr(out)) != TSP_OK)
    return s;
  if (out == attn || (attn_lo && out == attn_lo)) return TSP_ERR_INVALID_ARG;
  if (!workspace) return TSP_ERR_WORKSPACE;
  if (!aligned16(workspace)) return TSP_ERR_ALIGNMENT;
  if (ws_bytes < ws_out_shard(n_tokens, dims)) return TSP_ERR_WORKSPACE;
  if (n_tokens == 0) return TSP_OK;
  const int32_t ks = (dims->n_heads / D) * dims->head_dim;
  GemmArgs g{};
  g.A = attn + (int64_t)shard * ks;
  g.A_lo = attn_lo ? attn_lo + (int64_t)shard * ks : nullptr;
  g.lda = dims->hidden;
  g.B[0] = wo_d;
  g.M = (int32_t)n_tokens;
  g.N_s = dims->hidden;
  g.K_s = ks;
  g.n_shards = 1;
  g.k_shards = 1;
  g.epilogue = EPI_RESID;
  g.ldo = dims->hidden;
  ring_io(g, D, pos, residual, out, static_cast<float*>(workspace), 0, dims->hidden);
  return from_hip(launch_gemm(g, stream));
}

tsp_status tsp_mlp_shard(int64_t n_tokens, const tsp_dims* dims, int32_t D, int32_t pos, const uint16_t* x,
                         const uint16_t* w1_d, const uint16_t* w2_d, const uint16_t* residual, uint16_t* y,
                         void* workspace, size_t ws_bytes, hipStream_t stream) {
  tsp_status s;
  if ((s = check_dims(dims, D, false, true)) != TSP_OK) return s;
  if (n_tokens < 0) return TSP_ERR_SHAPE;
  if (n_tokens > INT32_MAX) return TSP_ERR_UNSUPPORTED;
  if (pos < 0 || pos >= D) return TSP_ERR_INVALID_ARG;
  if ((s = check_ptr(x)) != TSP_OK || (s = check_ptr(w1_d)) != TSP_OK || (s = check_ptr(w2_d)) != TSP_OK ||
      (s = check_ptr_nullable(residual)) != TSP_OK || (s = check_ptr(y)) != TSP_OK)
    return s;
  if (y == x) return TSP_ERR_INVALID_ARG;
  if (!workspace) return TSP_ERR_WORKSPACE;
  if (!aligned16(workspace)) return TSP_ERR_ALIGNMENT;
  const MlpShardWs lay = mlp_shard_ws(n_tokens, dims, D);
  if (ws_bytes < lay.total) return TSP_ERR_WORKSPACE;
  if (n_tokens == 0) return TSP_OK;
  char* base = static_cast<char*>(workspace);
  float* acc = reinterpret_cast<float*>(base + lay.acc_off);
  int32_t* row_exp = reinterpret_cast<int32_t*>(base + lay.exp_off);
  uint16_t* w2h = reinterpret_cast<uint16_t*>(base + lay.w2_off);
  uint16_t* hbuf = reinterpret_cast<uint16_t*>(base + lay.h_off);
  const int64_t h = dims->hidden;
  const int32_t fs = dims->ffn / D;
  if (pos == 0 && (s = from_hip(launch_row_prep(x, 0, n_tokens, dims->hidden, row_exp, nullptr, stream))) != TSP_OK)
    return s;
  const uint16_t* w2_one[1] = {w2_d};
  if ((s = from_hip(launch_bf16_to_f16(w2_one, w2h, 1, h * fs, stream))) != TSP_OK) return s;
  for (int64_t b0 = 0; b0 < n_tokens; b0 += MLP_TOKEN_BLOCK) {
    const int64_t mb = (n_tokens - b0) < MLP_TOKEN_BLOCK ? (n_tokens - b0) : MLP_TOKEN_BLOCK;
    GemmArgs g1{};
    g1.A = x + b0 * h;
    g1.lda = h;
    g1.B[0] = w1_d;
    g1.M = (int32_t)mb;
    g1.N_s = fs;
    g1.K_s = (int32_t)h;
    g1.n_shards = 1;
    g1.k_shards = 1;
    g1.epilogue = EPI_GELU;
    g1.out = hbuf;
    g1.ldo = fs;
    g1.row_exp = row_exp + b0;
    if ((s = from_hip(launch_gemm(g1, stream))) != TSP_OK) return s;
    GemmArgs g2{};
    g2.f16 = 1;
    g2.A = hbuf;
    g2.lda = fs;
    g2.B[0] = w2h;
    g2.M = (int32_t)mb;
    g2.N_s = (int32_t)h;
    g2.K_s = fs;
    g2.n_shards = 1;
    g2.k_shards = 1;
    g2.epilogue = EPI_RESID;
    g2.ldo = h;
    g2.row_exp = row_exp + b0;
    ring_io(g2, D, pos, residual, y, acc, b0, h);
    if ((s = from_hip(launch_gemm(g2, stream))) != TSP_OK) return s;
  }
  return TSP_OK;
}

// ---- layer variants ------------------------------------------------------------

tsp_status tsp_attn_project_arrival(const tsp_plan* plan, const tsp_dims* dims, int32_t start_shard,
                                    const uint16_t* x_local, const uint16_t* const* wqkv, uint16_t* k_full,
                                    uint16_t* v_full, uint16_t* q_out, const tsp_arrival* arrival,
                                    hipStream_t stream) {
  tsp_status s;
  if ((s = check_plan(plan)) != TSP_OK) return s;
  if ((s = check_dims(dims, plan->D, true, false)) != TSP_OK) return s;
  if (start_shard < 0 || start_shard >= plan->D) return TSP_ERR_INVALID_ARG;
  if ((s = check_ptr(x_local)) != TSP_OK || (s = check_shards(wqkv, plan->D)) != TSP_OK ||
      (s = check_ptr(k_full)) != TSP_OK || (s = check_ptr(v_full)) != TSP_OK || (s = check_ptr(q_out)) != TSP_OK ||
      (s = check_arrival(arrival)) != TSP_OK)
    return s;
  return run_project(plan, dims, x_local, wqkv, k_full, v_full, q_out, stream, start_shard, arrival);
}

tsp_status tsp_attn_out_arrival(int64_t n_tokens, const tsp_dims* dims, int32_t D, int32_t start_shard,
                                const uint16_t* attn, const uint16_t* attn_lo, const uint16_t* const* wo,
                                const uint16_t* residual, uint16_t* out, const tsp_arrival* arrival,
                                hipStream_t stream) {
  tsp_status s;
  if ((s = check_dims(dims, D, true, false)) != TSP_OK) return s;
  if (n_tokens < 0) return TSP_ERR_SHAPE;
  if (n_tokens > INT32_MAX) return TSP_ERR_UNSUPPORTED;
  if (start_shard < 0 || start_shard >= D) return TSP_ERR_INVALID_ARG;
  if ((s = check_ptr(attn)) != TSP_OK || (s = check_ptr_nullable(attn_lo)) != TSP_OK ||
      (s = check_shards(wo, D)) != TSP_OK || (s = check_ptr_nullable(residual)) != TSP_OK ||
      (s = check_ptr(out)) != TSP_OK || (s = check_arrival(arrival)) != TSP_OK)
    return s;
  if (out == attn || (attn_lo && out == attn_lo)) return TSP_ERR_INVALID_ARG;
  return run_out(n_tokens, dims, D, start_shard, attn, attn_lo, wo, residual, out, false, stream, arrival);
}

tsp_status tsp_mlp_forward_arrival(int64_t n_tokens, const tsp_dims* dims, int32_t D, int32_t start_shard,
                                   const uint16_t* x, const uint16_t* const* w1, const uint16_t* const* w2,
                                   const uint16_t* residual, uint16_t* y, void* workspace, size_t ws_bytes,
                                   const tsp_arrival* arrival, hipStream_t stream) {
  tsp_status s;
  if ((s = check_dims(dims, D, false, true)) != TSP_OK) return s;
  if (n_tokens < 0) return TSP_ERR_SHAPE;
  if (n_tokens > INT32_MAX) return TSP_ERR_UNSUPPORTED;
  if (start_shard < 0 || start_shard >= D) return TSP_ERR_INVALID_ARG;
  if ((s = check_ptr(x)) != TSP_OK || (s = check_shards(w1, D)) != TSP_OK || (s = check_shards(w2, D)) != TSP_OK ||
      (s = check_ptr_nullable(residual)) != TSP_OK || (s = check_ptr(y)) != TSP_OK ||
      (s = check_arrival(arrival)) != TSP_OK)
    return s;
  if (y == x && residual != x) return TSP_ERR_INVALID_ARG;
  if (!workspace) return TSP_ERR_WORKSPACE;
  if (!aligned16(workspace)) return TSP_ERR_ALIGNMENT;
  if (ws_bytes < ws_mlp(n_tokens, dims)) return TSP_ERR_WORKSPACE;
  if (n_tokens == 0) return TSP_OK;
  return run_mlp(n_tokens, dims, D, start_shard, x, w1, w2, residual, y, workspace, stream, arrival);
}

tsp_status tsp_simulate_arrival(int32_t n, const void* const* src, void* const* dst, const size_t* bytes,
                                uint32_t* counter, uint32_t base, uint32_t delay_us, hipStream_t stream) {
  if (n < 0 || n > ARRIVAL_MAX || delay_us > 1000000u || !counter) return TSP_ERR_INVALID_ARG;
  if ((uintptr_t)counter & 3u) return TSP_ERR_ALIGNMENT;
  if (n > 0 && (!src || !dst || !bytes)) return TSP_ERR_INVALID_ARG;
  ArrivalCopies c{};
  for (int32_t i = 0; i < n; ++i) {
    tsp_status s;
    if ((s = check_ptr(src[i])) != TSP_OK || (s = check_ptr(dst[i])) != TSP_OK) return s;
    if (bytes[i] % 16 != 0) return TSP_ERR_SHAPE;
    c.src[i] = src[i];
    c.dst[i] = dst[i];
    c.bytes[i] = bytes[i];
  }
  return from_hip(launch_simulate_arrival(c, n, counter, base, (uint64_t)delay_us * 100u, stream));
}

tsp_status tsp_rms_norm(int64_t n_tokens, int32_t hidden, const uint16_t* x, const uint16_t* gain, float eps,
                        uint16_t* y, hipStream_t stream) {
  tsp_status s;
  if (n_tokens < 0 || hidden <= 0) return TSP_ERR_SHAPE;
  if (hidden % 8 != 0) return TSP_ERR_UNSUPPORTED;
  if (!(eps >= 0.0f) || !(eps < 1.0e30f)) return TSP_ERR_INVALID_ARG;
  if ((s = check_ptr(x)) != TSP_OK || (s = check_ptr(gain)) != TSP_OK || (s = check_ptr(y)) != TSP_OK) return s;
  return from_hip(launch_rms_norm(x, gain, n_tokens, hidden, eps, y, stream));
}

tsp_status tsp_rope(const tsp_plan* plan, int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, double theta,
                    uint16_t* q, uint16_t* k_full, hipStream_t stream) {
  tsp_status s;
  if ((s = check_plan(plan)) != TSP_OK) return s;
  if (n_heads <= 0 || n_kv_heads <= 0 || head_dim <= 0) return TSP_ERR_SHAPE;
  if (head_dim % 8 != 0) return TSP_ERR_UNSUPPORTED;
  if (!(theta > 1.0) || !(theta < 1.0e300)) return TSP_ERR_INVALID_ARG;
  if ((s = check_ptr_nullable(q)) != TSP_OK || (s = check_ptr_nullable(k_full)) != TSP_OK) return s;
  if (q && (s = from_hip(launch_rope(q, 0, 0, plan->n_local, (int64_t)n_heads * head_dim, n_heads, head_dim, theta,
                                     plan->chunk_len, plan->chunk_start[0], plan->chunk_start[1], 0, stream))) != TSP_OK)
    return s;
  if (k_full)
    return from_hip(launch_rope(k_full, 0, 0, plan->n_local, (int64_t)n_kv_heads * head_dim, n_kv_heads, head_dim,
                                theta, plan->chunk_len, plan->chunk_start[0], plan->chunk_start[1], 1, stream));
  return TSP_OK;
}

tsp_status tsp_rope_backward(const tsp_plan* plan, int32_t n_heads, int32_t n_kv_heads, int32_t head_dim,
                             double theta, float* dq, float* dk_own, hipStream_t stream) {
  tsp_status s;
  if ((s = check_plan(plan)) != TSP_OK) return s;
  if (n_heads <= 0 || n_kv_heads <= 0 || head_dim <= 0) return TSP_ERR_SHAPE;
  if (head_dim % 8 != 0) return TSP_ERR_UNSUPPORTED;
  if (!(theta > 1.0) || !(theta < 1.0e300)) return TSP_ERR_INVALID_ARG;
  if ((s = check_ptr_nullable(dq)) != TSP_OK || (s = check_ptr_nullable(dk_own)) != TSP_OK) return s;
  if (dq && (void*)dq == (void*)dk_own) return TSP_ERR_INVALID_ARG;
  if (dq && (s = from_hip(launch_rope(dq, 1, 1, plan->n_local, (int64_t)n_heads * head_dim, n_heads, head_dim, theta,
                                      plan->chunk_len, plan->chunk_start[0], plan->chunk_start[1], 0, stream))) != TSP_OK)
    return s;
  if (dk_own)
    return from_hip(launch_rope(dk_own, 1, 1, plan->n_local, (int64_t)n_kv_heads * head_dim, n_kv_heads, head_dim,
                                theta, plan->chunk_len, plan->chunk_start[0], plan->chunk_start[1], 0, stream));
  return TSP_OK;
}

tsp_status tsp_rms_norm_backward(int64_t n_tokens, int32_t hidden, const uint16_t* x, const uint16_t* gain, float eps,
                                 const uint16_t* dy, uint16_t* dx, float* dgain, void* workspace, size_t ws_bytes,
                                 hipStream_t stream) {
  tsp_status s;
  if (n_tokens < 0 || hidden <= 0) return TSP_ERR_SHAPE;
  if (hidden % 8 != 0 || hidden > 8192) return TSP_ERR_UNSUPPORTED;
  if (!(eps >= 0.0f) || !(eps < 1.0e30f)) return TSP_ERR_INVALID_ARG;
  if ((s = check_ptr(gain)) != TSP_OK || (s = check_ptr(dgain)) != TSP_OK) return s;
  if (n_tokens == 0) return from_hip(launch_zero_f32(dgain, hidden, stream));  // token buffers are not used
  if ((s = check_ptr(x)) != TSP_OK || (s = check_ptr(dy)) != TSP_OK || (s = check_ptr(dx)) != TSP_OK) return s;
  if (dx == x || dx == dy) return TSP_ERR_INVALID_ARG;
  const size_t need = round_up((size_t)rms_norm_bwd_blocks(n_tokens) * hidden * 4);
  if (need > 0 && !workspace) return TSP_ERR_WORKSPACE;
  if (workspace && !aligned16(workspace)) return TSP_ERR_ALIGNMENT;
  if (ws_bytes < need) return TSP_ERR_WORKSPACE;
  return from_hip(launch_rms_norm_backward(x, gain, dy, n_tokens, hidden, eps, dx, dgain,
                                           static_cast<float*>(workspace), stream));
}

tsp_status tsp_attn_project_gqa(const tsp_plan* plan, const tsp_dims* dims, int32_t n_kv_heads,
                                const uint16_t* x_local, const uint16_t* const* wqkv, uint16_t* k_full,
                                uint16_t* v_full, uint16_t* q_out, hipStream_t stream) {
  tsp_status s;
  if ((s = check_plan(plan)) != TSP_OK) return s;
  if ((s = check_dims(dims, plan->D, true, false)) != TSP_OK) return s;
  if ((s = check_gqa(dims, plan->D, n_kv_heads, true)) != TSP_OK) return s;
  if ((s = check_ptr(x_local)) != TSP_OK || (s = check_shards(wqkv, plan->D)) != TSP_OK ||
      (s = check_ptr(k_full)) != TSP_OK || (s = check_ptr(v_full)) != TSP_OK || (s = check_ptr(q_out)) != TSP_OK)
    return s;
  GemmArgs g{};
  g.A = x_local;
  g.lda = dims->hidden;
  for (int d = 0; d < plan->D; ++d) g.B[d] = wqkv[d];
  const int hs = dims->n_heads / plan->D, kvs = n_kv_heads / plan->D;
  g.M = (int32_t)plan->n_local;
  g.N_s = (hs + 2 * kvs) * dims->head_dim;
  g.K_s = dims->hidden;
  g.n_shards = plan->D;
  g.k_shards = 1;
  g.epilogue = EPI_QKV;
  g.q_out = q_out;
  g.k_full = k_full;
  g.v_full = v_full;
  g.heads_per_shard = hs;
  g.kv_heads_per_shard = kvs;
  g.kv_ld = n_kv_heads * dims->head_dim;
  g.head_dim = dims->head_dim;
  g.hidden = dims->hidden;
  g.chunk_len = plan->chunk_len;
  g.chunk_start0 = plan->chunk_start[0];
  g.chunk_start1 = plan->chunk_start[1];
  return from_hip(launch_gemm(g, stream));
}

tsp_status tsp_attn_core_gqa(const tsp_plan* plan, const tsp_dims* dims, int32_t n_kv_heads, const uint16_t* q,
                             const uint16_t* k_full, const uint16_t* v_full, uint16_t* attn_out, uint16_t* attn_lo,
                             void* workspace, size_t ws_bytes, hipStream_t stream) {
  tsp_status s;
  if ((s = check_plan(plan)) != TSP_OK) return s;
  if ((s = check_dims(dims, plan->D, true, false, 0)) != TSP_OK) return s;
  if ((s = check_gqa(dims, plan->D, n_kv_heads, false)) != TSP_OK) return s;
  if ((s = check_ptr(q)) != TSP_OK || (s = check_ptr(k_full)) != TSP_OK || (s = check_ptr(v_full)) != TSP_OK ||
      (s = check_ptr(attn_out)) != TSP_OK || (s = check_ptr_nullable(attn_lo)) != TSP_OK)
    return s;
  if (attn_out == q || attn_lo == q || attn_lo == attn_out) return TSP_ERR_INVALID_ARG;
  if ((s = check_ws(workspace, ws_bytes, ws_core(plan->n_local, dims, plan->D))) != TSP_OK) return s;
  AttnArgs a{};
  a.q = q;
  a.k = k_full;
  a.v = v_full;
  a.o = attn_out;
  a.o_lo = attn_lo;
  a.seq_len = plan->seq_len;
  a.chunk_len = plan->chunk_len;
  a.chunk_start0 = plan->chunk_start[0];
  a.chunk_start1 = plan->chunk_start[1];
  a.hidden = dims->hidden;
  a.n_heads = dims->n_heads;
  a.head_dim = dims->head_dim;
  a.kv_heads = n_kv_heads;
  a.kv_ld = n_kv_heads * dims->head_dim;
  a.ws = workspace;
  return from_hip(launch_attention(a, stream));
}

tsp_status tsp_attn_core_gqa_lse(const tsp_plan* plan, const tsp_dims* dims, int32_t n_kv_heads, const uint16_t* q,
                                 const uint16_t* k_full, const uint16_t* v_full, uint16_t* attn_out,
                                 uint16_t* attn_lo, float* lse, void* workspace, size_t ws_bytes,
                                 hipStream_t stream) {
  tsp_status s;
  if ((s = check_ptr(lse)) != TSP_OK) return s;
  if ((s = check_plan(plan)) != TSP_OK) return s;
  if ((s = check_dims(dims, plan->D, true, false, 0)) != TSP_OK) return s;
  if ((s = check_gqa(dims, plan->D, n_kv_heads, false)) != TSP_OK) return s;
  if ((s = check_ptr(q)) != TSP_OK || (s = check_ptr(k_full)) != TSP_OK || (s = check_ptr(v_full)) != TSP_OK ||
      (s = check_ptr(attn_out)) != TSP_OK || (s = check_ptr_nullable(attn_lo)) != TSP_OK)
    return s;
  if (attn_out == q || attn_lo == q || attn_lo == attn_out) return TSP_ERR_INVALID_ARG;
  if ((s = check_ws(workspace, ws_bytes, ws_core(plan->n_local, dims, plan->D))) != TSP_OK) return s;
  AttnArgs a{};
  a.q = q;
  a.k = k_full;
  a.v = v_full;
  a.o = attn_out;
  a.o_lo = attn_lo;
  a.lse = lse;
  a.seq_len = plan->seq_len;
  a.chunk_len = plan->chunk_len;
  a.chunk_start0 = plan->chunk_start[0];
  a.chunk_start1 = plan->chunk_start[1];
  a.hidden = dims->hidden;
  a.n_heads = dims->n_heads;
  a.head_dim = dims->head_dim;
  a.kv_heads = n_kv_heads;
  a.kv_ld = n_kv_heads * dims->head_dim;
  a.ws = workspace;
  return from_hip(launch_attention(a, stream));
}

tsp_status tsp_attn_core_gqa_backward(const tsp_plan* plan, const tsp_dims* dims, int32_t n_kv_heads,
                                      const uint16_t* q, const uint16_t* k_full, const uint16_t* v_full,
                                      const uint16_t* attn_out, const uint16_t* attn_lo, const float* lse,
                                      const uint16_t* d_attn, float* dq, float* dk_full, float* dv_full,
                                      void* workspace, size_t ws_bytes, hipStream_t stream) {
  tsp_status s;
  if ((s = check_plan(plan)) != TSP_OK) return s;
  if ((s = check_dims(dims, plan->D, true, false, 0)) != TSP_OK) return s;
  if ((s = check_gqa(dims, plan->D, n_kv_heads, false)) != TSP_OK) return s;
  return run_attn_backward(plan, dims, n_kv_heads, q, k_full, v_full, attn_out, attn_lo, lse, d_attn, dq, dk_full,
                           dv_full, workspace, ws_bytes, stream);
}

tsp_status tsp_mlp_backward(int64_t n_tokens, const tsp_dims* dims, int32_t D, int32_t start_shard,
                            int32_t residual, const uint16_t* x, const uint16_t* const* w1,
                            const uint16_t* const* w2, const uint16_t* dy, uint16_t* dx, float* const* dw1,
                            float* const* dw2, void* workspace, size_t ws_bytes, hipStream_t stream) {
  tsp_status s;
  if ((s = check_dims(dims, D, false, true)) != TSP_OK) return s;
  if (n_tokens < 0) return TSP_ERR_SHAPE;
  if (n_tokens > INT32_MAX - 64) return TSP_ERR_UNSUPPORTED;
  if (start_shard < 0 || start_shard >= D) return TSP_ERR_INVALID_ARG;
  if ((s = check_shards(w1, D)) != TSP_OK || (s = check_shards(w2, D)) != TSP_OK) return s;
  if (!dw1 || !dw2) return TSP_ERR_INVALID_ARG;
  for (int d = 0; d < D; ++d)
    if ((s = check_ptr(dw1[d])) != TSP_OK || (s = check_ptr(dw2[d])) != TSP_OK) return s;
  if (n_tokens == 0) {  // no tokens: the weight gradients are zero; token buffers are not used
    const int64_t per = (int64_t)(dims->ffn / D) * dims->hidden;
    for (int d = 0; d < D; ++d)
      if ((s = from_hip(launch_zero_f32(dw1[d], per, stream))) != TSP_OK ||
          (s = from_hip(launch_zero_f32(dw2[d], per, stream))) != TSP_OK)
        return s;
    return TSP_OK;
  }
  if ((s = check_ptr(x)) != TSP_OK || (s = check_ptr(dy)) != TSP_OK || (s = check_ptr(dx)) != TSP_OK) return s;
  if (dx == x || dx == dy) return TSP_ERR_INVALID_ARG;
  if (!workspace) return TSP_ERR_WORKSPACE;
  if (!aligned16(workspace)) return TSP_ERR_ALIGNMENT;
  const MlpBwdWs lay = mlp_bwd_ws(n_tokens, dims, D);
  if (ws_bytes < lay.total) return TSP_ERR_WORKSPACE;
  char* base = static_cast<char*>(workspace);
  uint16_t* xt = reinterpret_cast<uint16_t*>(base + lay.xt_off);
  uint16_t* dyt = reinterpret_cast<uint16_t*>(base + lay.dyt_off);
  float* u = reinterpret_cast<float*>(base + lay.u_off);
  uint16_t* ht = reinterpret_cast<uint16_t*>(base + lay.ht_off);
  uint16_t* dut = reinterpret_cast<uint16_t*>(base + lay.dut_off);
  uint16_t* du = reinterpret_cast<uint16_t*>(base + lay.du_off);
  uint16_t* w1t = reinterpret_cast<uint16_t*>(base + lay.w1t_off);
  uint16_t* w2t = reinterpret_cast<uint16_t*>(base + lay.w2t_off);
  const int64_t n = n_tokens, np = pad64(n), h = dims->hidden, F = dims->ffn;
  const int32_t fs = dims->ffn / D;
  auto gemm = [&](const uint16_t* A, int64_t lda, const uint16_t* B, int32_t M, int32_t N, int32_t K, int epi,
                  void* out, int64_t ldo, int32_t out_f32) {
    GemmArgs g{};
    g.A = A;
    g.lda = lda;
    g.B[0] = B;
    g.M = M;
    g.N_s = N;
    g.K_s = K;
    g.n_shards = 1;
    g.k_shards = 1;
    g.epilogue = epi;
    g.out = out;
    g.ldo = ldo;
    g.out_f32 = out_f32;
    g.aux = u;
    return from_hip(launch_gemm(g, stream));
  };
  if ((s = from_hip(launch_transpose(x, 0, 0, n, h, h, xt, np, stream))) != TSP_OK) return s;
  if ((s = from_hip(launch_transpose(dy, 0, 0, n, h, h, dyt, np, stream))) != TSP_OK) return s;
  for (int k = 0; k < D; ++k) {
    const int d = (start_shard + k) % D;
    // U = x W1_d^T (fp32); GELU(U)^T; W2_d^T
    uint16_t* ht_d = ht + (int64_t)d * fs * np;
    uint16_t* dut_d = dut + (int64_t)d * fs * np;
    if ((s = gemm(x, h, w1[d], (int32_t)n, fs, (int32_t)h, EPI_RESID, u, fs, 1)) != TSP_OK) return s;
    if ((s = from_hip(launch_transpose(u, 1, 1, n, fs, fs, ht_d, np, stream))) != TSP_OK) return s;
    if ((s = from_hip(launch_transpose(w2[d], 0, 0, h, fs, fs, w2t, h, stream))) != TSP_OK) return s;
    // dU_d = (dy W2_d) * GELU'(U) -> block d of dU; its transpose
    if ((s = gemm(dy, h, w2t, (int32_t)n, fs, (int32_t)h, EPI_DGELU, du + (int64_t)d * fs, F, 0)) != TSP_OK) return s;
    if ((s = from_hip(launch_transpose(du + (int64_t)d * fs, 0, 0, n, fs, F, dut_d, np, stream))) != TSP_OK) return s;
    // W1_d^T for dx
    if ((s = from_hip(launch_transpose(w1[d], 0, 0, fs, h, h, w1t + (int64_t)d * h * fs, fs, stream))) != TSP_OK)
      return s;
  }
  // weight gradients of all shards in two launches (contractions over the tokens):
  // dW2_d = dy^T GELU(U_d) (N-sharded over the GELU(U)^T blocks) and
  // dW1_d = dU_d^T x (rows of dU^T in blocks of F_s), each into its own buffer
  {
    GemmArgs g{};
    g.A = dyt;
    g.lda = np;
    for (int d = 0; d < D; ++d) {
      g.B[d] = ht + (int64_t)d * fs * np;
      g.outs[d] = dw2[d];
    }
    g.M = (int32_t)h;
    g.N_s = fs;
    g.K_s = (int32_t)np;
    g.n_shards = D;
    g.k_shards = 1;
    g.epilogue = EPI_RESID;
    g.ldo = fs;
    g.out_f32 = 1;
    if ((s = from_hip(launch_gemm(g, stream))) != TSP_OK) return s;
  }
  {
    GemmArgs g{};
    g.A = dut;
    g.lda = np;
    g.B[0] = xt;
    for (int d = 0; d < D; ++d) g.outs[d] = dw1[d];
    g.rows_per_out = fs;
    g.M = (int32_t)F;
    g.N_s = (int32_t)h;
    g.K_s = (int32_t)np;
    g.n_shards = 1;
    g.k_shards = 1;
    g.epilogue = EPI_RESID;
    g.ldo = h;
    g.out_f32 = 1;
    if ((s = from_hip(launch_gemm(g, stream))) != TSP_OK) return s;
  }
  // dx = [dy +] sum_k dU[:, d_k block] W1_{d_k}: the ring's split-K, fp32 in registers
  GemmArgs g{};
  g.A = du;
  g.lda = F;
  for (int d = 0; d < D; ++d) g.B[d] = w1t + (int64_t)d * h * fs;
  g.M = (int32_t)n;
  g.N_s = (int32_t)h;
  g.K_s = fs;
  g.n_shards = 1;
  g.k_shards = D;
  g.ring_start = start_shard;
  g.epilogue = EPI_RESID;
  g.out = dx;
  g.ldo = h;
  g.residual = residual ? dy : nullptr;
  return from_hip(launch_gemm(g, stream));
}

tsp_status tsp_attn_out_backward(int64_t n_tokens, const tsp_dims* dims, int32_t D, int32_t start_shard,
                                 const uint16_t* attn, const uint16_t* const* wo, const uint16_t* d_out,
                                 uint16_t* d_attn, float* const* dwo, void* workspace, size_t ws_bytes,
                                 hipStream_t stream) {
  tsp_status s;
  if ((s = check_dims(dims, D, true, false)) != TSP_OK) return s;
  if (n_tokens < 0) return TSP_ERR_SHAPE;
  if (n_tokens > INT32_MAX - 64) return TSP_ERR_UNSUPPORTED;
  if (start_shard < 0 || start_shard >= D) return TSP_ERR_INVALID_ARG;
  if ((s = check_shards(wo, D)) != TSP_OK) return s;
  if (!dwo) return TSP_ERR_INVALID_ARG;
  for (int d = 0; d < D; ++d)
    if ((s = check_ptr(dwo[d])) != TSP_OK) return s;
  if (n_tokens == 0) {  // no tokens: the weight gradients are zero; token buffers are not used
    const int64_t per = (int64_t)(dims->n_heads / D) * dims->head_dim * dims->hidden;
    for (int d = 0; d < D; ++d)
      if ((s = from_hip(launch_zero_f32(dwo[d], per, stream))) != TSP_OK) return s;
    return TSP_OK;
  }
  if ((s = check_ptr(attn)) != TSP_OK || (s = check_ptr(d_out)) != TSP_OK || (s = check_ptr(d_attn)) != TSP_OK)
    return s;
  if (d_attn == attn || d_attn == d_out) return TSP_ERR_INVALID_ARG;
  if (!workspace) return TSP_ERR_WORKSPACE;
  if (!aligned16(workspace)) return TSP_ERR_ALIGNMENT;
  const OutBwdWs lay = out_bwd_ws(n_tokens, dims, D);
  if (ws_bytes < lay.total) return TSP_ERR_WORKSPACE;
  char* base = static_cast<char*>(workspace);
  uint16_t* wot = reinterpret_cast<uint16_t*>(base + lay.wot_off);
  uint16_t* dot = reinterpret_cast<uint16_t*>(base + lay.dot_off);
  uint16_t* at = reinterpret_cast<uint16_t*>(base + lay.at_off);
  const int64_t n = n_tokens, np = pad64(n), h = dims->hidden;
  const int32_t hs = (dims->n_heads / D) * dims->head_dim;
  if ((s = from_hip(launch_transpose(d_out, 0, 0, n, h, h, dot, np, stream))) != TSP_OK) return s;
  if ((s = from_hip(launch_transpose(attn, 0, 0, n, h, h, at, np, stream))) != TSP_OK) return s;
  for (int k = 0; k < D; ++k) {
    const int d = (start_shard + k) % D;
    if ((s = from_hip(launch_transpose(wo[d], 0, 0, h, hs, hs, wot + (int64_t)d * hs * h, h, stream))) != TSP_OK)
      return s;
  }
  // dW_o_d = d_out^T attn[:, block d] for every shard in one N-sharded launch
  // (contraction over the tokens), each into its own buffer
  {
    GemmArgs g{};
    g.A = dot;
    g.lda = np;
    for (int d = 0; d < D; ++d) {
      g.B[d] = at + (int64_t)d * hs * np;
      g.outs[d] = dwo[d];
    }
    g.M = (int32_t)h;
    g.N_s = hs;
    g.K_s = (int32_t)np;
    g.n_shards = D;
    g.k_shards = 1;
    g.epilogue = EPI_RESID;
    g.ldo = hs;
    g.out_f32 = 1;
    if ((s = from_hip(launch_gemm(g, stream))) != TSP_OK) return s;
  }
  // d_attn[:, block d] = d_out W_o_d: one N-sharded launch over the transposed shards
  GemmArgs g{};
  g.A = d_out;
  g.lda = h;
  for (int d = 0; d < D; ++d) g.B[d] = wot + (int64_t)d * hs * h;
  g.M = (int32_t)n;
  g.N_s = hs;
  g.K_s = (int32_t)h;
  g.n_shards = D;
  g.k_shards = 1;
  g.epilogue = EPI_RESID;
  g.out = d_attn;
  g.ldo = h;
  return from_hip(launch_gemm(g, stream));
}

tsp_status tsp_attn_project_backward(int64_t n_tokens, const tsp_dims* dims, int32_t D, int32_t start_shard,
                                     const uint16_t* x, const uint16_t* const* wqkv, const float* dq, const float* dk,
                                     const float* dv, const uint16_t* dy, uint16_t* dx, float* const* dwqkv,
                                     void* workspace, size_t ws_bytes, hipStream_t stream) {
  tsp_status s;
  if ((s = check_dims(dims, D, true, false)) != TSP_OK) return s;
  if (n_tokens < 0) return TSP_ERR_SHAPE;
  if (n_tokens > INT32_MAX - 64) return TSP_ERR_UNSUPPORTED;
  if (start_shard < 0 || start_shard >= D) return TSP_ERR_INVALID_ARG;
  if ((s = check_shards(wqkv, D)) != TSP_OK) return s;
  if (!dwqkv) return TSP_ERR_INVALID_ARG;
  for (int d = 0; d < D; ++d)
    if ((s = check_ptr(dwqkv[d])) != TSP_OK) return s;
  if (n_tokens == 0) {  // no tokens: the weight gradients are zero; token buffers are not used
    const int64_t per = (int64_t)3 * (dims->n_heads / D) * dims->head_dim * dims->hidden;
    for (int d = 0; d < D; ++d)
      if ((s = from_hip(launch_zero_f32(dwqkv[d], per, stream))) != TSP_OK) return s;
    return TSP_OK;
  }
  if ((s = check_ptr(x)) != TSP_OK || (s = check_ptr(dq)) != TSP_OK || (s = check_ptr(dk)) != TSP_OK ||
      (s = check_ptr(dv)) != TSP_OK || (s = check_ptr_nullable(dy)) != TSP_OK || (s = check_ptr(dx)) != TSP_OK)
    return s;
  if (dx == x) return TSP_ERR_INVALID_ARG;
  if (!workspace) return TSP_ERR_WORKSPACE;
  if (!aligned16(workspace)) return TSP_ERR_ALIGNMENT;
  const ProjBwdWs lay = proj_bwd_ws(n_tokens, dims, D);
  if (ws_bytes < lay.total) return TSP_ERR_WORKSPACE;
  char* base = static_cast<char*>(workspace);
  uint16_t* G = reinterpret_cast<uint16_t*>(base + lay.g_off);
  uint16_t* xt = reinterpret_cast<uint16_t*>(base + lay.xt_off);
  uint16_t* gt = reinterpret_cast<uint16_t*>(base + lay.gt_off);
  uint16_t* wt = reinterpret_cast<uint16_t*>(base + lay.wt_off);
  const int64_t n = n_tokens, np = pad64(n), h = dims->hidden;
  const int32_t hs = (dims->n_heads / D) * dims->head_dim;
  const float* parts[3] = {dq, dk, dv};
  for (int p = 0; p < 3; ++p)
    if ((s = from_hip(launch_f32_to_bf16(parts[p], n, h, h, G + p * h, 3 * h, stream))) != TSP_OK) return s;
  if ((s = from_hip(launch_transpose(x, 0, 0, n, h, h, xt, np, stream))) != TSP_OK) return s;
  for (int k = 0; k < D; ++k) {
    const int d = (start_shard + k) % D;
    // [dq_d | dk_d | dv_d]^T into block d of G^T
    for (int p = 0; p < 3; ++p)
      if ((s = from_hip(launch_transpose(parts[p] + (int64_t)d * hs, 1, 0, n, hs, h,
                                         gt + ((int64_t)d * 3 + p) * hs * np, np, stream))) != TSP_OK)
        return s;
    // the shard's Q, K and V weight blocks transposed, [h x H_s*hd] each
    for (int p = 0; p < 3; ++p)
      if ((s = from_hip(launch_transpose(wqkv[d] + (int64_t)p * hs * h, 0, 0, hs, h, h,
                                         wt + ((int64_t)p * D + d) * h * hs, hs, stream))) != TSP_OK)
        return s;
  }
  // dW_qkv_d = G^T block d . x for every shard in one launch (rows of G^T in
  // blocks of 3 H_s*hd; contraction over the tokens), each into its own buffer
  {
    GemmArgs g{};
    g.A = gt;
    g.lda = np;
    g.B[0] = xt;
    for (int d = 0; d < D; ++d) g.outs[d] = dwqkv[d];
    g.rows_per_out = 3 * hs;
    g.M = 3 * (int32_t)h;
    g.N_s = (int32_t)h;
    g.K_s = (int32_t)np;
    g.n_shards = 1;
    g.k_shards = 1;
    g.epilogue = EPI_RESID;
    g.ldo = h;
    g.out_f32 = 1;
    if ((s = from_hip(launch_gemm(g, stream))) != TSP_OK) return s;
  }
  // dx = [dy +] sum_p sum_d G_p[:, block d] W_{p, d}: one split-K over the 3D
  // blocks (K-shard j = p*D + d sits at columns j*H_s*hd of G, its weight
  // block at slot j of the transposed weights), one fp32 accumulator in
  // registers, blocks visited from j = start_shard round to start_shard - 1
  GemmArgs g{};
  g.A = G;
  g.lda = 3 * h;
  for (int j = 0; j < 3 * D; ++j) g.B[j] = wt + (int64_t)j * h * hs;
  g.M = (int32_t)n;
  g.N_s = (int32_t)h;
  g.K_s = hs;
  g.n_shards = 1;
  g.k_shards = 3 * D;
  g.ring_start = start_shard;
  g.epilogue = EPI_RESID;
  g.ldo = h;
  g.residual = dy;
  g.out = dx;
  return from_hip(launch_gemm(g, stream));
}

tsp_status tsp_memory_footprint(int64_t seq_len, const tsp_dims* dims, int32_t D, int32_t n_layers,
                                int32_t scheme, int32_t training, tsp_memory* out) {
  if (!out || !dims || n_layers < 0) return TSP_ERR_INVALID_ARG;
  if (scheme != TSP_MEM_TSP && scheme != TSP_MEM_TP) return TSP_ERR_INVALID_ARG;
  tsp_status s = check_dims(dims, D, true, true);
  if (s != TSP_OK) return s;
  tsp_plan plan;
  if ((s = tsp_zigzag_plan(seq_len, D, 0, &plan, nullptr, nullptr)) != TSP_OK) return s;

  const uint64_t h = (uint64_t)dims->hidden, F = (uint64_t)dims->ffn, S = (uint64_t)seq_len;
  const uint64_t layer_params = 4 * h * h + 2 * h * F;  // W_q, W_k, W_v, W_o; W1, W2
  const uint64_t own_params = (uint64_t)n_layers * layer_params / (uint64_t)D;
  const bool tsp = scheme == TSP_MEM_TSP;
  const uint64_t tokens = tsp ? (uint64_t)plan.n_local : S;

  tsp_memory m{};
  m.weights = own_params * 2;
  m.streamed = tsp && n_layers > 0 ? (uint64_t)(D - 1) * (layer_params / (uint64_t)D) * 2 : 0;
  if (tsp) {
    m.kv = 2 * S * h * 2;
    m.activations = 2 * round_up(tokens * h * 2) + ws_layer((int64_t)tokens, dims, D);
  } else {
    // The buffers of tsp_layer_forward (input and output rows, Q, attention
    // output hi and lo, the attention core's workspace, fp32 h1, its scaled
    // fp16 copy, row exponents, fp16 W1 and W2 copies, one GELU token block)
    // for all S tokens, with the rank's H/D heads and F/D FFN columns.
    const uint64_t wa = h / (uint64_t)D, wf = F / (uint64_t)D;
    const uint64_t mb = tokens < (uint64_t)MLP_TOKEN_BLOCK ? tokens : (uint64_t)MLP_TOKEN_BLOCK;
    m.kv = 2 * S * wa * 2;
    m.activations = 2 * round_up(tokens * h * 2) + 3 * round_up(tokens * wa * 2) +
                    round_up(attn_core_workspace((int64_t)S, (int64_t)S / 2, (int32_t)wa, dims->n_heads / D)) +
                    round_up(tokens * h * 4) + round_up(tokens * h * 2) + round_up(tokens * 4) +
                    2 * round_up(wf * h * 2) + round_up(mb * wf * 2);
  }
  if (training) {
    m.train_state = own_params * 14 + (uint64_t)n_layers * tokens * h * 2;
    m.grads = n_layers > 0 ? (tsp ? layer_params : layer_params / (uint64_t)D) * 4 : 0;
  }
  if (n_layers == 0) m.kv = m.activations = 0;
  m.total = m.weights + m.streamed + m.kv + m.activations + m.train_state + m.grads;
  *out = m;
  return TSP_OK;
}

const char* tsp_status_string(tsp_status status) {
  switch (status) {
    case TSP_OK: return "TSP_OK";
    case TSP_ERR_INVALID_ARG: return "TSP_ERR_INVALID_ARG: null pointer, bad enum or out-of-range index";
    case TSP_ERR_SHAPE: return "TSP_ERR_SHAPE: shapes inconsistent with the zigzag plan or the layer";
    case TSP_ERR_ALIGNMENT: return "TSP_ERR_ALIGNMENT: device pointer not 16-byte aligned";
    case TSP_ERR_WORKSPACE: return "TSP_ERR_WORKSPACE: workspace missing or too small";
    case TSP_ERR_UNSUPPORTED: return "TSP_ERR_UNSUPPORTED: head_dim or width not supported by the kernels";
    case TSP_ERR_HIP: return "TSP_ERR_HIP: a kernel launch failed";
    case TSP_ERR_SCRATCH: return "TSP_ERR_SCRATCH: more scratch than the allocation-free entry point's fixed array";
    default: return "TSP: unknown status";
  }
}

}  // extern "C"
