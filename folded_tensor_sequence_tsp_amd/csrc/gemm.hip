// Shard-iterated bf16 GEMM engine for gfx950 (CDNA4) on v_mfma_f32_32x32x16_bf16.
//
// C = A . B^T with both operands K-contiguous (weights stored out x in).  The
// weight operand arrives as D separate shards, the way TSP hands them to a
// device one after another (zubnet.ai, "Zyphra TSP folds TP+SP onto one GPU
// axis", para. 2):
//   * N-sharded mode (QKV projection, MLP W1): shard d produces output column
//     block d; one launch covers all shards, a tile never straddles two.
//   * K-sharded mode (O projection, MLP W2): shard d contributes the partial
//     product of K block d; a tile walks the shards in ring order with one
//     fp32 accumulator held in registers, which is the local sum that stands
//     in for tensor parallelism's all-reduce.
//
// Tiling: BM x BN x 64 block tile, 256 threads = 4 waves in a 2 x 2 grid, each
// wave owning a (BM/2) x (BN/2) sub-tile of 32 x 32 MFMA tiles.  Global ->
// register prefetch of the next K tile overlaps the MFMAs of the current one;
// LDS is double-buffered (one barrier per K tile) and rows are padded by 16
// bytes so the 16-byte fragment reads of 8 consecutive rows hit disjoint banks.
// Workgroup ids are remapped so each XCD (ids = x mod 8) gets a contiguous run
// of tiles, then rasterised in groups of 8 tile rows for L2 reuse of B.
#include "device_common.h"
#include "kernels.h"

namespace tsp {
namespace {

constexpr int BK = 64;
constexpr int LDK = BK + 8;  // padded LDS row, bf16 elements (144 bytes)
constexpr int NTHREADS = 256;

template <int BM, int BN>
struct Cfg {
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int FM = WM / 32, FN = WN / 32;
  static constexpr int A_CHUNKS = BM * BK / 8 / NTHREADS;  // 16-byte chunks per thread
  static constexpr int B_CHUNKS = BN * BK / 8 / NTHREADS;
  static constexpr int LDS_ELEMS = 2 * (BM + BN) * LDK;
};

template <int EPI>
__device__ __forceinline__ void store_elem(const GemmArgs& g, int nshard, int row, int col, float acc) {
  if constexpr (EPI == EPI_RESID) {
    const int64_t idx = (int64_t)row * g.ldo + col;
    float v = acc;
    if (g.residual) v += bf16_to_f32(g.residual[idx]);
    g.out[idx] = f32_to_bf16(v);
  } else if constexpr (EPI == EPI_GELU) {
    g.out[(int64_t)row * g.ldo + (int64_t)nshard * g.N_s + col] = f32_to_bf16(gelu_tanh(acc));
  } else {
    const int hs_hd = g.heads_per_shard * g.head_dim;
    const int part = col / hs_hd;  // 0 = Q, 1 = K, 2 = V
    const int gcol = nshard * hs_hd + (col - part * hs_hd);
    const uint16_t b = f32_to_bf16(acc);
    if (part == 0) {
      g.q_out[(int64_t)row * g.hidden + gcol] = b;
    } else {
      const int64_t gpos = row < g.chunk_len ? g.chunk_start0 + row : g.chunk_start1 + (row - g.chunk_len);
      uint16_t* dst = part == 1 ? g.k_full : g.v_full;
      dst[gpos * g.hidden + gcol] = b;
    }
  }
}

template <int BM, int BN, int EPI>
__global__ __launch_bounds__(NTHREADS) void gemm_kernel(const GemmArgs g) {
  using C = Cfg<BM, BN>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::LDS_ELEMS];
  uint16_t* As = lds;                 // [2][BM][LDK]
  uint16_t* Bs = lds + 2 * BM * LDK;  // [2][BN][LDK]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  const int tiles_m = (g.M + BM - 1) / BM;
  const int tiles_n_shard = (g.N_s + BN - 1) / BN;
  const int tiles_n = tiles_n_shard * g.n_shards;
  const int nwg = gridDim.x;
  int pid = blockIdx.x;
  if ((nwg & 7) == 0) pid = (pid & 7) * (nwg >> 3) + (pid >> 3);
  constexpr int GROUP_M = 8;
  const int group_size = GROUP_M * tiles_n;
  const int first_m = (pid / group_size) * GROUP_M;
  const int gm = min(tiles_m - first_m, GROUP_M);
  const int in_group = pid % group_size;
  const int tm = first_m + in_group % gm;
  const int tn = in_group / gm;
  const int nshard = tn / tiles_n_shard;
  const int n0 = (tn - nshard * tiles_n_shard) * BN;
  const int m0 = tm * BM;

  const int kt_per_shard = g.K_s / BK;
  const int k_tiles = kt_per_shard * g.k_shards;

  // Per-thread load coordinates: chunk c = i*256 + tid -> row c/8, 16-byte column c%8.
  const int ld_row = tid >> 3;
  const int ld_kc = (tid & 7) * 8;
  constexpr int ROWS_PER_PASS = NTHREADS / 8;  // 32

  const uint16_t* a_rows[C::A_CHUNKS];
#pragma unroll
  for (int i = 0; i < C::A_CHUNKS; ++i) {
    const int r = min(m0 + i * ROWS_PER_PASS + ld_row, g.M - 1);
    a_rows[i] = g.A + (int64_t)r * g.lda + ld_kc;
  }
  int64_t b_off[C::B_CHUNKS];
#pragma unroll
  for (int i = 0; i < C::B_CHUNKS; ++i) {
    const int n = min(n0 + i * ROWS_PER_PASS + ld_row, g.N_s - 1);
    b_off[i] = (int64_t)n * g.K_s + ld_kc;
  }

  u32x4 ra[C::A_CHUNKS], rb[C::B_CHUNKS];
  auto load_tile = [&](int t) {
    const int s = t / kt_per_shard;
    const int kt = t - s * kt_per_shard;
    int d;
    int64_t acol;
    if (g.k_shards > 1) {
      d = g.ring_start + s;
      if (d >= g.k_shards) d -= g.k_shards;
      acol = (int64_t)d * g.K_s + kt * BK;
    } else {
      d = nshard;
      acol = kt * BK;
    }
    const uint16_t* bp = g.B[d] + kt * BK;
#pragma unroll
    for (int i = 0; i < C::A_CHUNKS; ++i) ra[i] = *reinterpret_cast<const u32x4*>(a_rows[i] + acol);
#pragma unroll
    for (int i = 0; i < C::B_CHUNKS; ++i) rb[i] = *reinterpret_cast<const u32x4*>(bp + b_off[i]);
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::A_CHUNKS; ++i)
      *reinterpret_cast<u32x4*>(As + (buf * BM + i * ROWS_PER_PASS + ld_row) * LDK + ld_kc) = ra[i];
#pragma unroll
    for (int i = 0; i < C::B_CHUNKS; ++i)
      *reinterpret_cast<u32x4*>(Bs + (buf * BN + i * ROWS_PER_PASS + ld_row) * LDK + ld_kc) = rb[i];
  };

  f32x16 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc[i][j] = f32x16{};

  const int frag_row = lane & 31;
  const int frag_k = (lane >> 5) * 8;

  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int t = 0; t < k_tiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < k_tiles) load_tile(t + 1);
    const uint16_t* a_base = As + (buf * BM + wm * C::WM + frag_row) * LDK + frag_k;
    const uint16_t* b_base = Bs + (buf * BN + wn * C::WN + frag_row) * LDK + frag_k;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 af[C::FM], bfv[C::FN];
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
        af[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(a_base + i * 32 * LDK + kk * 16));
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
        bfv[j] = as_bf16x8(*reinterpret_cast<const u32x4*>(b_base + j * 32 * LDK + kk * 16));
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) acc[i][j] = mfma32(af[i], bfv[j], acc[i][j]);
    }
    if (t + 1 < k_tiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // Epilogue.  32x32 accumulator layout: lane holds column (lane % 32) and rows
  // 8*(e/4) + 4*(lane/32) + e%4 for its 16 values e.
  const int col_l = lane & 31;
  const int row_l = 4 * (lane >> 5);
#pragma unroll
  for (int i = 0; i < C::FM; ++i) {
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      const int col = n0 + wn * C::WN + j * 32 + col_l;
      if (col >= g.N_s) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + wm * C::WM + i * 32 + 8 * (e >> 2) + row_l + (e & 3);
        if (row < g.M) store_elem<EPI>(g, nshard, row, col, acc[i][j][e]);
      }
    }
  }
}

template <int BM, int BN>
hipError_t launch_tiles(const GemmArgs& g, hipStream_t stream) {
  const int tiles_m = (g.M + BM - 1) / BM;
  const int tiles_n = ((g.N_s + BN - 1) / BN) * g.n_shards;
  const dim3 grid(tiles_m * tiles_n), block(NTHREADS);
  switch (g.epilogue) {
    case EPI_QKV: hipLaunchKernelGGL((gemm_kernel<BM, BN, EPI_QKV>), grid, block, 0, stream, g); break;
    case EPI_GELU: hipLaunchKernelGGL((gemm_kernel<BM, BN, EPI_GELU>), grid, block, 0, stream, g); break;
    default: hipLaunchKernelGGL((gemm_kernel<BM, BN, EPI_RESID>), grid, block, 0, stream, g); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& g, hipStream_t stream) {
  if (g.M <= 0) return hipSuccess;
  // 256 x 256 tiles keep the LDS traffic per MFMA low; fall back to 128 x 128
  // when the big tiles would leave most of the 256 CUs idle.
  const long big = (long)((g.M + 255) / 256) * (((g.N_s + 255) / 256) * g.n_shards);
  if (big >= 192) return launch_tiles<256, 256>(g, stream);
  return launch_tiles<128, 128>(g, stream);
}

}  // namespace tsp
