// Internal launch interface between the C-ABI layer (tsp_api.cpp) and the HIP
// kernels (gemm.hip, attention.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "../../include/tsp.h"

namespace tsp {

enum GemmEpilogue : int32_t {
  EPI_QKV = 0,    // Q -> q_out, K/V rows -> k_full/v_full at global zigzag positions (bf16)
  EPI_GELU = 1,   // out[:, shard block] = fp16(GELU(acc * 2^in_exp) * 2^-row_exp[row])
  EPI_RESID = 2,  // out = (acc * 2^row_exp[row] [+ residual]) as bf16 or fp32
  EPI_DGELU = 3,  // out[:, shard block] = bf16(acc * GELU'(aux[row, col])), aux fp32 [M x N_s]
};

// C = A . B^T over 16-bit operands (bf16, or fp16 when f16 is set) with an fp32
// accumulator.
//  N-sharded ("column") mode, k_shards == 1: output columns come in n_shards
//    blocks of N_s; block d uses B[d] ([N_s x K_s]); A is [M x K_s].
//  K-sharded ("split-K") mode, n_shards == 1: B[d] is [N_s x K_s] and A is
//    [M x k_shards*K_s]; shards are visited in ring order
//    (ring_start + s) mod k_shards with one accumulator.
// row_exp (nullable = all 0) holds a power-of-two exponent per output row:
//  EPI_GELU scales its fp16 output by 2^-row_exp (and, when gelu_in_scaled, the
//  accumulator by 2^+row_exp before GELU: the A rows were stored scaled);
//  EPI_RESID scales the accumulator by 2^+row_exp before the residual.
struct GemmArgs {
  int32_t f16;  // operands are fp16 (else bf16)
  const uint16_t* A;
  // Optional low part of A (bf16 residual of A's rounding, same layout): each
  // shard's K range is then contracted twice against the same B columns, once
  // with A and once with A_lo, into the same accumulator.
  const uint16_t* A_lo;
  int64_t lda;
  const uint16_t* B[3 * TSP_MAX_D];  // up to 3*D K-shards: a split-K over the Q, K and V parts of D shards
  int32_t M, N_s, K_s;
  int32_t n_shards, k_shards, ring_start;
  int32_t epilogue;
  // EPI_GELU / EPI_RESID
  void* out;
  int64_t ldo;
  // EPI_RESID into separate buffers (out unused): when outs[0] is set, an
  // N-sharded launch writes shard s's columns to outs[s] (columns from 0), and
  // a launch with rows_per_out > 0 writes rows [k*rows_per_out, (k+1)*rows_per_out)
  // to outs[k] (rows from 0); row stride ldo in both.
  void* outs[TSP_MAX_D];
  int32_t rows_per_out;
  const float* aux;       // EPI_DGELU: the GELU inputs, fp32, row stride N_s
  const void* residual;  // EPI_RESID, nullable
  int32_t res_f32;       // residual is fp32 (else bf16)
  int32_t out_f32;       // EPI_RESID output is fp32 (else bf16)
  const int32_t* row_exp;
  int32_t gelu_in_scaled;
  // EPI_QKV
  uint16_t* q_out;
  uint16_t* k_full;
  uint16_t* v_full;
  int32_t heads_per_shard, head_dim, hidden;
  int32_t shard0;  // index of the launch's first weight shard (its Q/K/V column block)
  // grouped-query projection: K/V heads per shard and the row stride of k_full /
  // v_full (0: as many as the query heads, stride hidden)
  int32_t kv_heads_per_shard, kv_ld;
  int64_t chunk_len, chunk_start0, chunk_start1;
  // Shard arrival (nullable `arrived`): a shard is read only once
  // (int32_t)(*arrived - arrived_base) exceeds its ring position (K-sharded:
  // the count of shards walked before it from ring_start; N-sharded shard s:
  // (s - ring_start) mod n_shards).  Wave 0 of a workgroup polls the counter
  // with system-scope loads at the tile's first load and at each later shard
  // not yet known to have arrived; a wait that has polled spin_limit times
  // sets *arrival_status = 1 and the tile goes on as if everything had arrived.
  const uint32_t* arrived;
  uint32_t arrived_base, spin_limit;
  uint32_t* arrival_status;
};

// hipErrorInvalidValue when 256 rows of A (lda) or of a B shard (K_s) span
// more than 2^31 bytes (the loads address a tile through one buffer
// descriptor with 32-bit offsets): lda, K_s < 4,194,304 elements.
hipError_t launch_gemm(const GemmArgs& args, hipStream_t stream);

// Simulated shard arrival on one workgroup: for i = 0..n-1, wait until
// (i + 1) * delay_ticks of the 100 MHz wall clock have passed since the kernel
// started, copy bytes[i] (a multiple of 16) from src[i] to dst[i], write the
// copy back to memory, then store base + i + 1 into *counter (system scope).
constexpr int ARRIVAL_MAX = 64;
struct ArrivalCopies {
  const void* src[ARRIVAL_MAX];
  void* dst[ARRIVAL_MAX];
  uint64_t bytes[ARRIVAL_MAX];
};
hipError_t launch_simulate_arrival(const ArrivalCopies& c, int32_t n, uint32_t* counter, uint32_t base,
                                   uint64_t delay_ticks, hipStream_t stream);

// For each row i of x [n x h] (fp32 when x_f32, else bf16):
//   row_exp[i] = floor(log2(rms of the row)) (0 for a zero or non-finite rms),
//   and, when x16 is not null, x16[i] = fp16(x[i] * 2^-row_exp[i]) (saturated).
hipError_t launch_row_prep(const void* x, int32_t x_f32, int64_t n, int32_t h, int32_t* row_exp, uint16_t* x16,
                           hipStream_t stream);

// dst[d] = fp16(src[d]) for D shards of `count` bf16 elements each (count % 8 == 0);
// values beyond the fp16 range saturate to +-65504.
hipError_t launch_bf16_to_f16(const uint16_t* const* src, uint16_t* dst, int32_t D, int64_t count,
                              hipStream_t stream);

struct AttnArgs {
  const uint16_t* q;  // [n_local x hidden]
  const uint16_t* k;  // [seq_len x kv_ld]
  const uint16_t* v;  // [seq_len x kv_ld]
  uint16_t* o;        // [n_local x hidden]
  uint16_t* o_lo;     // nullable: bf16(out - o), the rounding residual of o
  int64_t seq_len, chunk_len, chunk_start0, chunk_start1;
  int32_t hidden, n_heads, head_dim;
  // K/V heads (n_heads for MHA; fewer for grouped-query attention, query head a
  // reading K/V head a / (n_heads / kv_heads)) and the row stride of k and v.
  int32_t kv_heads, kv_ld;
  // workspace of attn_core_workspace() bytes (nullable when that is 0)
  void* ws;
  // nullable: lse[head * 2 * chunk_len + row] = ln sum_j exp(score), the
  // natural log of each query row's softmax normaliser (kept for the backward).
  float* lse;
  // set by launch_attention when it splits the late chunk's keys in two
  // (in the workspace): the halves' unnormalised outputs
  // [2][chunk_len][hidden] fp32 and (max in log2 units, sum) pairs
  // [2][n_heads][chunk_len][2]
  float* part_o;
  float* part_ml;
};

// Attention tiling shared by the kernel and the host-side sizes: queries per
// workgroup, keys per tile, and the grid size below which the late chunk's
// key range is split in two.
constexpr int ATTN_QT = 256;
constexpr int ATTN_BKV = 64;
constexpr int64_t ATTN_SPLIT_BELOW = 512;

// 256-byte rounding of the workspace parts.
constexpr size_t attn_align(size_t x) { return (x + 255) / 256 * 256; }

// Whether launch_attention splits the late chunk's key range (few query tiles).
bool attn_split(int64_t chunk_len, int32_t n_heads);

// 64-key tiles covering seq_len keys.
int64_t attn_kv_tiles(int64_t seq_len);

// Bytes of workspace launch_attention needs: the split partials when the grid
// is small, else none.
size_t attn_core_workspace(int64_t seq_len, int64_t chunk_len, int32_t hidden, int32_t n_heads);

// The attention kernel (and, for split grids, the combine kernel) on `stream`.
hipError_t launch_attention(const AttnArgs& args, hipStream_t stream);

// Rows [0, rows) of src (row stride ld, head h in columns h*head_dim ..) ->
// transposed 64-row tiles dst[((h * n_tiles + t) * head_dim + d) * 64 + k] =
// src[t*64 + perm16(k)][h*head_dim + d], zero past `rows`; the rows of each
// 16-row group in the order (bits 2 and 3 of the index swapped) in which a
// 32x32 MFMA result holds them.  Grid (n_tiles, heads).
hipError_t launch_vt_tiles(const uint16_t* src, int64_t rows, int32_t ld, int32_t heads, int32_t head_dim,
                           uint16_t* dst, int64_t n_tiles, hipStream_t stream);

// p[0 .. count) = 0 (a kernel, not a memset, so that the call can be captured).
hipError_t launch_zero_f32(float* p, int64_t count, hipStream_t stream);

// dst[r * ld_out + c] = bf16(src[r * ld_in + c]) for r < R, c < C (C % 8 == 0).
hipError_t launch_f32_to_bf16(const float* src, int64_t R, int64_t C, int64_t ld_in, uint16_t* dst, int64_t ld_out,
                              hipStream_t stream);

// Backward of the causal attention of the two zigzag chunks (MHA).
struct AttnBwdArgs {
  const uint16_t* q;     // [n_local x hidden]
  const uint16_t* k;     // [seq_len x hidden]
  const uint16_t* v;     // [seq_len x hidden]
  const uint16_t* o;     // [n_local x hidden], the forward's output
  const uint16_t* o_lo;  // nullable: its low part
  const uint16_t* dout;  // [n_local x hidden]
  const float* lse;      // [n_heads x n_local], natural log of each row's softmax normaliser
  float* dq;             // [n_local x hidden]
  float* dk;             // [seq_len x hidden]: this rank's contributions, every key row
  float* dv;             // [seq_len x hidden]
  int64_t seq_len, chunk_len, chunk_start0, chunk_start1;
  int32_t hidden, n_heads, head_dim;
  // K/V heads (n_heads for MHA; grouped-query: query head a reads K/V head
  // a / (n_heads / kv_heads)) and the row stride of k, v, dk, dv.
  int32_t kv_heads, kv_ld;
  // workspace (kt, qt, dot at head_dim 64 only; null otherwise): K^T tiles
  // [H_kv][n_kv_tiles][hd][64]; Q^T and dO^T tiles [2 chunks][H][tpc][hd][64];
  // per 64-query tile of (chunk, head) 256 floats: log2-domain normaliser
  // [64], delta = rowsum(dO * O) [64], zeros [128].
  uint16_t* kt;
  uint16_t* qt;
  uint16_t* dot;
  float* stats;
  int64_t n_kv_tiles, tpc;  // 64-key tiles of the sequence; 64-query tiles per chunk
};

// Whether the dK/dV kernel streams pre-transposed Q^T and dO^T tiles (head_dim
// 64) rather than reading the row-major Q and dO tiles with transposing LDS
// reads (head_dim 128); the workspace holds those tiles only in the first case.
constexpr bool attn_bwd_stages_qt(int head_dim) { return head_dim != 128; }
// Likewise for the dQ kernel's K^T tiles.
constexpr bool attn_bwd_stages_kt(int head_dim) { return head_dim != 128; }
// Workspace bytes of launch_attention_backward.
size_t attn_bwd_ws_bytes(int64_t seq_len, int64_t chunk_len, int32_t n_heads, int32_t kv_heads, int32_t head_dim);

// Pre-passes (stats; K^T, Q^T, dO^T tiles at head_dim 64), then the dK/dV and dQ kernels.
hipError_t launch_attention_backward(const AttnBwdArgs& args, hipStream_t stream);

// y = x / sqrt(mean(x^2) + eps) * gain per row of x [n x h] (bf16; h % 8 == 0).
hipError_t launch_rms_norm(const uint16_t* x, const uint16_t* gain, int64_t n, int32_t h, float eps, uint16_t* y,
                           hipStream_t stream);

// Rotary embedding in place of the n_rows local rows (positions from the zigzag
// chunks), n_heads heads of head_dim each, row stride ld: rows of x itself, or
// (at_global) the rows of x at the global positions.
// x_f32: the rows are fp32 (else bf16); inverse: rotate by -angle (the backward).
hipError_t launch_rope(void* x, int32_t x_f32, int32_t inverse, int64_t n_rows, int64_t ld, int32_t n_heads,
                       int32_t head_dim, double theta, int64_t chunk_len, int64_t start0, int64_t start1,
                       int32_t at_global, hipStream_t stream);

// Rows per workgroup of the RMSNorm backward (its partial dgain rows).
constexpr int RMS_BWD_ROWS = 32;

// Backward of RMSNorm over x [n x h] (bf16, h % 8 == 0, h <= 8192): dx (bf16)
// and dgain (fp32 [h]); partial: fp32 [rms_norm_bwd_blocks(n) x h] scratch.
int64_t rms_norm_bwd_blocks(int64_t n);
hipError_t launch_rms_norm_backward(const uint16_t* x, const uint16_t* gain, const uint16_t* dy, int64_t n,
                                    int32_t h, float eps, uint16_t* dx, float* dgain, float* partial,
                                    hipStream_t stream);

// dst[c * ld_out + r] = f(src[r * ld_in + c]) for r < R, c < C (C % 64 == 0), and 0
// for R <= r < ld_out (ld_out % 64 == 0): a transpose of bf16 (src_f32: fp32)
// rows into bf16, f = GELU (tanh form) when gelu, else the identity.
hipError_t launch_transpose(const void* src, int32_t src_f32, int32_t gelu, int64_t R, int64_t C, int64_t ld_in,
                            uint16_t* dst, int64_t ld_out, hipStream_t stream);

}  // namespace tsp
