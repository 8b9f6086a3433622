// Internal launch interface between the C-ABI layer (tsp_api.cpp) and the HIP
// kernels (gemm.hip, attention.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "../../include/tsp.h"

namespace tsp {

enum GemmEpilogue : int32_t {
  EPI_QKV = 0,    // Q -> q_out, K/V rows -> k_full/v_full at global zigzag positions
  EPI_GELU = 1,   // out[:, shard block] = bf16(GELU(acc))
  EPI_RESID = 2,  // out = bf16(acc [+ residual])
};

// C = A . B^T over bf16 operands with an fp32 accumulator.
//  N-sharded ("column") mode, k_shards == 1: output columns come in n_shards
//    blocks of N_s; block d uses B[d] ([N_s x K_s]); A is [M x K_s].
//  K-sharded ("split-K") mode, n_shards == 1: B[d] is [N_s x K_s] and A is
//    [M x k_shards*K_s]; shards are visited in ring order
//    (ring_start + s) mod k_shards with one accumulator.
struct GemmArgs {
  const uint16_t* A;
  int64_t lda;
  const uint16_t* B[TSP_MAX_D];
  int32_t M, N_s, K_s;
  int32_t n_shards, k_shards, ring_start;
  int32_t epilogue;
  // EPI_GELU / EPI_RESID
  uint16_t* out;
  int64_t ldo;
  const uint16_t* residual;  // EPI_RESID, nullable
  // EPI_QKV
  uint16_t* q_out;
  uint16_t* k_full;
  uint16_t* v_full;
  int32_t heads_per_shard, head_dim, hidden;
  int64_t chunk_len, chunk_start0, chunk_start1;
};

hipError_t launch_gemm(const GemmArgs& args, hipStream_t stream);

struct AttnArgs {
  const uint16_t* q;  // [n_local x hidden]
  const uint16_t* k;  // [seq_len x hidden]
  const uint16_t* v;  // [seq_len x hidden]
  uint16_t* o;        // [n_local x hidden]
  int64_t seq_len, chunk_len, chunk_start0, chunk_start1;
  int32_t hidden, n_heads, head_dim;
};

hipError_t launch_attention(const AttnArgs& args, hipStream_t stream);

}  // namespace tsp
