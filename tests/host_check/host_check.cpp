// Host-only driver of the C-ABI layer for the sanitizer build (tests/host_check):
// tsp_api.cpp and layout.cpp are compiled with AddressSanitizer and
// UndefinedBehaviorSanitizer and linked against recording launch stand-ins
// (stubs.cpp).  Every public entry point is called on buffers sized exactly as
// include/tsp.h documents them, over shapes that reach the planner's, the
// validation's and the workspace arithmetic's edge cases (D = 1 and
// TSP_MAX_D, ragged chunks, head_dim 64 and 128, split and unsplit attention
// grids, grouped-query heads, zero tokens); the stand-ins check that every
// kernel's byte ranges stay inside those buffers.  Invalid arguments must
// return their status and launch nothing.  Exit status 0 means all passed.
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "registry.h"
#include "tsp.h"

namespace {

int g_calls = 0, g_total_launches = 0;

void fail(const char* what, tsp_status s) {
  fprintf(stderr, "host_check: %s: status %d (%s)\n", what, (int)s, tsp_status_string(s));
  exit(1);
}

// A call that must succeed and (with work to do) launch kernels.
void ok(tsp_status s, const char* what, bool launches = true) {
  ++g_calls;
  if (s != TSP_OK) fail(what, s);
  if (launches && hc_launches() == 0) fail(what, s);
  g_total_launches += hc_launches();
  hc_reset_launches();
}

// A call that must be rejected with `want` and launch nothing.
void rejects(tsp_status s, tsp_status want, const char* what) {
  ++g_calls;
  if (s != want || hc_launches() != 0) {
    fprintf(stderr, "host_check: %s: status %d, expected %d, %d launches\n", what, (int)s, (int)want, hc_launches());
    exit(1);
  }
}

uint16_t* bf(size_t elems) { return static_cast<uint16_t*>(hc_alloc(elems * 2)); }
float* f32(size_t elems) { return static_cast<float*>(hc_alloc(elems * 4)); }
void* ws(size_t bytes) { return bytes ? hc_alloc(bytes) : nullptr; }

struct Shape {
  int32_t h, H, hd, F;
  int64_t S;
  int32_t D;
  int32_t kv;  // K/V heads of the grouped-query calls (0: skip them)
};

void layer_calls(const Shape& sh, int32_t r) {
  tsp_dims dims{sh.h, sh.H, sh.hd, sh.F};
  const int32_t D = sh.D;
  tsp_plan plan;
  std::vector<int64_t> l2g((size_t)(sh.S / D));
  std::vector<int32_t> ring(D);
  ok(tsp_zigzag_plan(sh.S, D, r, &plan, l2g.data(), ring.data()), "plan", false);
  const int64_t n = plan.n_local, S = sh.S, h = sh.h;
  const int64_t Hs = sh.H / D, hs_hd = Hs * sh.hd, Fs = sh.F / D;
  // layer tensors
  uint16_t* x = bf(n * h);
  uint16_t *wqkv[TSP_MAX_D], *wo[TSP_MAX_D], *w1[TSP_MAX_D], *w2[TSP_MAX_D];
  for (int d = 0; d < D; ++d) {
    wqkv[d] = bf(3 * hs_hd * h);
    wo[d] = bf(h * hs_hd);
    w1[d] = bf(Fs * h);
    w2[d] = bf(h * Fs);
  }
  uint16_t *kf = bf(S * h), *vf = bf(S * h), *q = bf(n * h), *a = bf(n * h), *alo = bf(n * h), *out = bf(n * h);
  float* lse = f32((size_t)sh.H * n);
  const auto sz = [&](int kind) { return tsp_workspace_size(n, &dims, D, kind); };
  void* w_core = ws(sz(TSP_WS_CORE));
  ok(tsp_attn_project(&plan, &dims, x, wqkv, kf, vf, q, 0), "attn_project");
  ok(tsp_attn_core(&plan, &dims, q, kf, vf, a, alo, w_core, sz(TSP_WS_CORE), 0), "attn_core");
  ok(tsp_attn_core(&plan, &dims, q, kf, vf, a, nullptr, w_core, sz(TSP_WS_CORE), 0), "attn_core no lo");
  ok(tsp_attn_core_lse(&plan, &dims, q, kf, vf, a, alo, lse, w_core, sz(TSP_WS_CORE), 0), "attn_core_lse");
  ok(tsp_attn_out(n, &dims, D, r, a, alo, wo, x, out, 0), "attn_out");
  ok(tsp_attn_out(n, &dims, D, r, a, nullptr, wo, nullptr, out, 0), "attn_out no lo, no residual");
  ok(tsp_attn_forward(&plan, &dims, x, wqkv, wo, kf, vf, x, out, ws(sz(TSP_WS_ATTN)), sz(TSP_WS_ATTN), 0),
     "attn_forward");
  ok(tsp_mlp_forward(n, &dims, D, r, x, w1, w2, nullptr, out, ws(sz(TSP_WS_MLP)), sz(TSP_WS_MLP), 0), "mlp_forward");
  ok(tsp_mlp_forward(n, &dims, D, r, x, w1, w2, x, out, ws(sz(TSP_WS_MLP)), sz(TSP_WS_MLP), 0), "mlp_forward resid");
  ok(tsp_layer_post(n, &dims, D, r, a, alo, x, wo, w1, w2, out, ws(sz(TSP_WS_POST)), sz(TSP_WS_POST), 0),
     "layer_post");
  ok(tsp_layer_forward(&plan, &dims, x, wqkv, wo, w1, w2, kf, vf, out, ws(sz(TSP_WS_LAYER)), sz(TSP_WS_LAYER), 0),
     "layer_forward");
  // shards awaited inside the kernels, and the simulated producer
  uint32_t* cnt = reinterpret_cast<uint32_t*>(f32(1));
  uint32_t* st = reinterpret_cast<uint32_t*>(f32(1));
  const tsp_arrival arr{cnt, 0u, 0u, st};
  ok(tsp_attn_project_arrival(&plan, &dims, r, x, wqkv, kf, vf, q, &arr, 0), "attn_project_arrival");
  ok(tsp_attn_out_arrival(n, &dims, D, r, a, alo, wo, x, out, &arr, 0), "attn_out_arrival");
  ok(tsp_mlp_forward_arrival(n, &dims, D, r, x, w1, w2, x, out, ws(sz(TSP_WS_MLP)), sz(TSP_WS_MLP), &arr, 0),
     "mlp_forward_arrival");
  {
    const void* src[TSP_MAX_D];
    void* dst[TSP_MAX_D];
    size_t nb[TSP_MAX_D];
    for (int d = 0; d < D; ++d) {
      src[d] = wo[d];
      dst[d] = bf(h * hs_hd);
      nb[d] = (size_t)h * hs_hd * 2;
    }
    ok(tsp_simulate_arrival(D, src, dst, nb, cnt, 0u, 10u, 0), "simulate_arrival");
  }
  // shard streaming: one ring
  void* w_os = ws(sz(TSP_WS_OUT_SHARD));
  void* w_ms = ws(sz(TSP_WS_MLP_SHARD));
  for (int pos = 0; pos < D; ++pos) {
    const int s = ring[pos];
    ok(tsp_attn_project_shard(&plan, &dims, s, x, wqkv[s], kf, vf, q, 0), "attn_project_shard");
    ok(tsp_attn_out_shard(n, &dims, D, pos, s, a, alo, wo[s], x, out, w_os, sz(TSP_WS_OUT_SHARD), 0), "attn_out_shard");
    ok(tsp_mlp_shard(n, &dims, D, pos, x, w1[s], w2[s], nullptr, out, w_ms, sz(TSP_WS_MLP_SHARD), 0), "mlp_shard");
  }
  // backward
  uint16_t *dy = bf(n * h), *dx = bf(n * h), *dattn = bf(n * h), *dattn2 = bf(n * h);
  float *dw1[TSP_MAX_D], *dw2[TSP_MAX_D], *dwo[TSP_MAX_D], *dwqkv[TSP_MAX_D];
  for (int d = 0; d < D; ++d) {
    dw1[d] = f32(Fs * h);
    dw2[d] = f32(h * Fs);
    dwo[d] = f32(h * hs_hd);
    dwqkv[d] = f32(3 * hs_hd * h);
  }
  ok(tsp_mlp_backward(n, &dims, D, r, 1, x, w1, w2, dy, dx, dw1, dw2, ws(sz(TSP_WS_MLP_BWD)), sz(TSP_WS_MLP_BWD), 0),
     "mlp_backward");
  ok(tsp_mlp_backward(0, &dims, D, r, 0, nullptr, w1, w2, nullptr, nullptr, dw1, dw2, nullptr, 0, 0),
     "mlp_backward, no tokens");
  float *dq = f32(n * h), *dk = f32(S * h), *dv = f32(S * h);
  ok(tsp_attn_core_backward(&plan, &dims, q, kf, vf, a, alo, lse, dattn, dq, dk, dv, ws(sz(TSP_WS_ATTN_BWD)),
                            sz(TSP_WS_ATTN_BWD), 0),
     "attn_core_backward");
  ok(tsp_attn_out_backward(n, &dims, D, r, a, wo, dy, dattn2, dwo, ws(sz(TSP_WS_OUT_BWD)), sz(TSP_WS_OUT_BWD), 0),
     "attn_out_backward");
  ok(tsp_attn_out_backward(0, &dims, D, r, nullptr, wo, nullptr, nullptr, dwo, nullptr, 0, 0),
     "attn_out_backward, no tokens");
  float *dqn = f32(n * h), *dkn = f32(n * h), *dvn = f32(n * h);
  ok(tsp_attn_project_backward(n, &dims, D, r, x, wqkv, dqn, dkn, dvn, dy, dx, dwqkv, ws(sz(TSP_WS_PROJ_BWD)),
                               sz(TSP_WS_PROJ_BWD), 0),
     "attn_project_backward");
  ok(tsp_attn_project_backward(n, &dims, D, r, x, wqkv, dqn, dkn, dvn, nullptr, dx, dwqkv, ws(sz(TSP_WS_PROJ_BWD)),
                               sz(TSP_WS_PROJ_BWD), 0),
     "attn_project_backward, no dy");
  ok(tsp_attn_project_backward(0, &dims, D, r, nullptr, wqkv, nullptr, nullptr, nullptr, nullptr, nullptr, dwqkv,
                               nullptr, 0, 0),
     "attn_project_backward, no tokens");
  // variants
  uint16_t* gain = bf(h);
  ok(tsp_rms_norm(n, sh.h, x, gain, 1e-6f, out, 0), "rms_norm");
  ok(tsp_rms_norm(n, sh.h, out, gain, 1e-6f, out, 0), "rms_norm in place");
  ok(tsp_rope(&plan, sh.H, sh.H, sh.hd, 1e4, q, kf, 0), "rope");
  ok(tsp_rope_backward(&plan, sh.H, sh.H, sh.hd, 1e4, dqn, dkn, 0), "rope_backward");
  const size_t rms_ws = tsp_workspace_size(n, &dims, 1, TSP_WS_RMS_BWD);
  float* dgain = f32(h);
  ok(tsp_rms_norm_backward(n, sh.h, x, gain, 1e-6f, dy, dx, dgain, ws(rms_ws), rms_ws, 0), "rms_norm_backward");
  ok(tsp_rms_norm_backward(0, sh.h, nullptr, gain, 1e-6f, nullptr, nullptr, dgain, nullptr, 0, 0),
     "rms_norm_backward, no tokens");
  if (sh.kv) {  // grouped-query attention
    const int64_t kvw = (int64_t)sh.kv * sh.hd, kvs = (int64_t)(sh.kv / D) * sh.hd;
    uint16_t *kg = bf(S * kvw), *vg = bf(S * kvw), *wg[TSP_MAX_D];
    for (int d = 0; d < D; ++d) wg[d] = bf((hs_hd + 2 * kvs) * h);
    ok(tsp_attn_project_gqa(&plan, &dims, sh.kv, x, wg, kg, vg, q, 0), "attn_project_gqa");
    ok(tsp_attn_core_gqa(&plan, &dims, sh.kv, q, kg, vg, a, alo, w_core, sz(TSP_WS_CORE), 0), "attn_core_gqa");
    ok(tsp_attn_core_gqa_lse(&plan, &dims, sh.kv, q, kg, vg, a, alo, lse, w_core, sz(TSP_WS_CORE), 0),
       "attn_core_gqa_lse");
    ok(tsp_rope(&plan, sh.H, sh.kv, sh.hd, 1e4, q, kg, 0), "rope gqa");
    float *dkg = f32(S * kvw), *dvg = f32(S * kvw);
    ok(tsp_attn_core_gqa_backward(&plan, &dims, sh.kv, q, kg, vg, a, alo, lse, dattn, dq, dkg, dvg,
                                  ws(sz(TSP_WS_ATTN_BWD)), sz(TSP_WS_ATTN_BWD), 0),
       "attn_core_gqa_backward");
  }
  // memory accounting
  tsp_memory m;
  for (int scheme = 0; scheme < 2; ++scheme)
    for (int training = 0; training < 2; ++training)
      ok(tsp_memory_footprint(S, &dims, D, 32, scheme, training, &m), "memory_footprint", false);
  hc_free_all();
}

void rejections() {
  tsp_dims dims{256, 4, 64, 1024};
  tsp_plan plan;
  ok(tsp_zigzag_plan(2048, 4, 1, &plan, nullptr, nullptr), "plan", false);
  const int64_t n = plan.n_local;
  uint16_t *x = bf(n * 256), *kf = bf(2048 * 256), *vf = bf(2048 * 256), *q = bf(n * 256), *a = bf(n * 256);
  uint16_t *w[TSP_MAX_D], *mis = x + 1;
  for (int d = 0; d < TSP_MAX_D; ++d) w[d] = bf(256 * 256);
  rejects(tsp_zigzag_plan(2047, 4, 1, &plan, nullptr, nullptr), TSP_ERR_SHAPE, "plan S % 2D");
  rejects(tsp_zigzag_plan(0, 4, 0, &plan, nullptr, nullptr), TSP_ERR_SHAPE, "plan S = 0");
  rejects(tsp_zigzag_plan(2048, 0, 0, &plan, nullptr, nullptr), TSP_ERR_INVALID_ARG, "plan D = 0");
  rejects(tsp_zigzag_plan(2048, TSP_MAX_D + 1, 0, &plan, nullptr, nullptr), TSP_ERR_INVALID_ARG, "plan D > max");
  rejects(tsp_zigzag_plan(2048, 4, 4, &plan, nullptr, nullptr), TSP_ERR_INVALID_ARG, "plan rank = D");
  rejects(tsp_zigzag_plan(2048, 4, -1, &plan, nullptr, nullptr), TSP_ERR_INVALID_ARG, "plan rank < 0");
  rejects(tsp_zigzag_plan(2048, 4, 0, nullptr, nullptr, nullptr), TSP_ERR_INVALID_ARG, "plan null");
  rejects(tsp_zigzag_plan((int64_t)1 << 62, 2, 0, &plan, nullptr, nullptr), TSP_ERR_UNSUPPORTED, "plan n > int32");
  ok(tsp_zigzag_plan(2048, 4, 1, &plan, nullptr, nullptr), "plan", false);
  rejects(tsp_attn_project(&plan, &dims, mis, w, kf, vf, q, 0), TSP_ERR_ALIGNMENT, "project misaligned x");
  rejects(tsp_attn_project(&plan, &dims, nullptr, w, kf, vf, q, 0), TSP_ERR_INVALID_ARG, "project null x");
  tsp_dims bad = dims;
  bad.head_dim = 32;
  bad.n_heads = 8;
  rejects(tsp_attn_project(&plan, &bad, x, w, kf, vf, q, 0), TSP_ERR_UNSUPPORTED, "project head_dim 32");
  bad = dims;
  bad.hidden = 320;
  rejects(tsp_attn_project(&plan, &bad, x, w, kf, vf, q, 0), TSP_ERR_SHAPE, "project hidden != H hd");
  tsp_plan forged = plan;
  forged.chunk_start[1] += 64;
  rejects(tsp_attn_project(&forged, &dims, x, w, kf, vf, q, 0), TSP_ERR_SHAPE, "project forged plan");
  rejects(tsp_attn_core(&plan, &dims, q, kf, vf, q, nullptr, nullptr, 0, 0), TSP_ERR_INVALID_ARG, "core out = q");
  const size_t need = tsp_workspace_size(n, &dims, 4, TSP_WS_CORE);
  void* w_core = ws(need);
  rejects(tsp_attn_core(&plan, &dims, q, kf, vf, a, nullptr, w_core, need - 1, 0), TSP_ERR_WORKSPACE,
          "core short workspace");
  rejects(tsp_attn_core(&plan, &dims, q, kf, vf, a, nullptr, nullptr, need, 0), TSP_ERR_WORKSPACE,
          "core null workspace");
  rejects(tsp_attn_out(n, &dims, 4, 4, a, nullptr, w, nullptr, q, 0), TSP_ERR_INVALID_ARG, "out start = D");
  rejects(tsp_attn_out(-1, &dims, 4, 0, a, nullptr, w, nullptr, q, 0), TSP_ERR_SHAPE, "out n < 0");
  rejects(tsp_attn_out(n, &dims, 4, 0, a, nullptr, w, nullptr, a, 0), TSP_ERR_INVALID_ARG, "out aliases attn");
  bad = dims;
  bad.ffn = 1002;
  rejects(tsp_mlp_forward(n, &bad, 4, 0, x, w, w, nullptr, q, nullptr, 0, 0), TSP_ERR_SHAPE, "mlp ffn % D");
  bad.ffn = 4 * 96;
  rejects(tsp_mlp_forward(n, &bad, 4, 0, x, w, w, nullptr, q, w_core, need, 0), TSP_ERR_UNSUPPORTED,
          "mlp ffn/D % 64");
  const size_t mneed = tsp_workspace_size(n, &dims, 4, TSP_WS_MLP);
  rejects(tsp_mlp_forward(n, &dims, 4, 0, x, w, w, nullptr, q, ws(mneed), mneed - 1, 0), TSP_ERR_WORKSPACE,
          "mlp short workspace");
  rejects(tsp_mlp_shard(n, &dims, 4, 4, x, w[0], w[0], nullptr, q, ws(mneed), mneed, 0), TSP_ERR_INVALID_ARG,
          "mlp_shard pos = D");
  rejects(tsp_attn_project_shard(&plan, &dims, 4, x, w[0], kf, vf, q, 0), TSP_ERR_INVALID_ARG, "project_shard = D");
  rejects(tsp_rms_norm(n, 260, x, w[0], 1e-6f, q, 0), TSP_ERR_UNSUPPORTED, "rms_norm hidden % 8");
  rejects(tsp_rms_norm(n, 256, x, w[0], -1.0f, q, 0), TSP_ERR_INVALID_ARG, "rms_norm eps < 0");
  rejects(tsp_rope(&plan, 4, 4, 64, 1.0, q, kf, 0), TSP_ERR_INVALID_ARG, "rope theta 1");
  rejects(tsp_attn_core_gqa(&plan, &dims, 3, q, kf, vf, a, nullptr, w_core, need, 0), TSP_ERR_SHAPE, "gqa 3 heads");
  tsp_memory m;
  rejects(tsp_memory_footprint(2048, &dims, 4, 1, 2, 0, &m), TSP_ERR_INVALID_ARG, "memory scheme");
  rejects(tsp_memory_footprint(2048, &dims, 4, -1, 0, 0, &m), TSP_ERR_INVALID_ARG, "memory n_layers");
  // workspace sizes: invalid kinds and dims give 0, huge token counts do not overflow into small sizes
  for (int kind = -1; kind <= 12; ++kind) {
    const size_t s = tsp_workspace_size(n, &dims, 4, kind);
    if ((kind < 0 || kind > 11) != (s == 0)) fail("workspace kind", TSP_ERR_INVALID_ARG);
  }
  bad = dims;
  bad.hidden = 300;
  if (tsp_workspace_size(n, &bad, 4, TSP_WS_LAYER) != 0) fail("workspace invalid dims", TSP_ERR_SHAPE);
  if (tsp_workspace_size(-1, &dims, 4, TSP_WS_LAYER) != 0) fail("workspace n < 0", TSP_ERR_SHAPE);
  if (tsp_workspace_size((int64_t)1 << 30, &dims, 4, TSP_WS_LAYER) < ((size_t)1 << 30) * 256 * 2)
    fail("workspace for 2^30 tokens", TSP_ERR_SHAPE);
  for (int st = -1; st <= 7; ++st)
    if (!tsp_status_string((tsp_status)st)) fail("status string", TSP_ERR_INVALID_ARG);
  hc_free_all();
}

}  // namespace

int main() {
  // (hidden, heads, head_dim, ffn, S, D, gqa K/V heads)
  const Shape shapes[] = {
      {256, 4, 64, 1024, 2048, 4, 0},     // the tiny layer: split attention grid
      {256, 4, 64, 1024, 520, 4, 0},      // ragged chunks of 65
      {512, 4, 128, 2048, 4096, 2, 2},    // head_dim 128, grouped-query (2 K/V heads)
      {1024, 16, 64, 1024, 2048, TSP_MAX_D, 0},  // D = TSP_MAX_D
      {256, 4, 64, 256, 512, 1, 2},       // D = 1
      {2048, 32, 64, 2048, 8192, 2, 0},   // an attention grid too large to split
  };
  for (const Shape& sh : shapes)
    for (int32_t r : {0, sh.D - 1}) layer_calls(sh, r);
  // every zigzag plan over a grid: exact cover of 0..S-1 by the D ranks
  for (int32_t D = 1; D <= TSP_MAX_D; ++D)
    for (int64_t C : {1, 3, 64, 65}) {
      const int64_t S = 2 * D * C;
      std::vector<int> seen((size_t)S, 0);
      for (int32_t r = 0; r < D; ++r) {
        tsp_plan p;
        std::vector<int64_t> l2g((size_t)(S / D));
        ok(tsp_zigzag_plan(S, D, r, &p, l2g.data(), nullptr), "plan grid", false);
        for (int64_t g : l2g) {
          if (g < 0 || g >= S) fail("plan position out of range", TSP_ERR_SHAPE);
          ++seen[(size_t)g];
        }
      }
      for (int c : seen)
        if (c != 1) fail("plan cover", TSP_ERR_SHAPE);
    }
  rejections();
  printf("host_check: %d calls, %d kernel launches checked\n", g_calls, g_total_launches);
  return 0;
}
