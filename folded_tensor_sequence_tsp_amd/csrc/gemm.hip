// Shard-iterated 16-bit GEMM engine for gfx950 (CDNA4) on v_mfma_f32_32x32x16_{bf16,f16}.
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
// Tiling: BM x BN x 64 block tile; waves of WM x WN (256 x 256 tiles: eight
// waves of 128 x 64, two per SIMD; 256 x 192 tiles, for QKV shards whose
// width is a multiple of 192 when they fill the rounds of tiles better:
// eight waves of 64 x 96; 128 x 256 tiles: eight waves of 64 x 64, for short
// token counts; 128 x 128 tiles: four waves of 64 x 64), each a grid of
// 32 x 32 MFMA tiles.  A and B k-tiles stream into an LDS ring with direct
// buffer->LDS loads (buffer_load_dwordx4 ... lds, no register staging; one
// descriptor pair per shard, the k-tile's column in the loads' scalar offset),
// one vmcnt wait and one barrier per k-tile: 256 x 256 tiles have two 64 KB
// stages (the other stage is refilled right after the barrier, before the
// MFMAs), 256 x 192 two of 56 KB, 128 x 256 three, 128 x 128 four.  Shard widths that are not a
// multiple of 64, and the O projection's two-part A, use 32-k tiles in a
// 4-stage (3 with two parts) ring.  Buffer rather than global loads: the
// compiler counts a global->LDS load against the LDS counter as well, so with
// loads always in flight every fragment wait became a wait for all of them;
// with buffer loads the waits are graduated.  LDS rows are 128 bytes (64 k
// values; 64 bytes for 32-k tiles); the 16-byte chunk c of row r sits at c ^
// ((r / 2) % 8) (c ^ ((r / 4) % 4)), so the 16 lanes of one LDS cycle, reading
// 16 consecutive rows at one k offset, hit distinct banks of the 64-bank LDS.
// Workgroup ids are remapped so each XCD (ids = x mod 8) gets a contiguous run
// of tiles, then rasterised in groups of 8 (QKV) or 4 tile rows for L2 reuse.
// With a low part of A (the O projection contracts the attention output's two
// bf16 parts), A and A_lo share each k-tile: a stage holds three tiles, each B
// fragment feeds two MFMAs, and the ring is three stages deep.
#include "device_common.h"
#include "kernels.h"

namespace tsp {
namespace {

constexpr int STAGES = 4;    // LDS ring depth of 32-k tiles
#ifndef GEMM_K64_DEFAULT
#define GEMM_K64_DEFAULT 1
#endif
constexpr bool GEMM_K64 = GEMM_K64_DEFAULT;

// LO: the low part of A (A_lo) shares each k-tile with A: a stage holds the
// A, A_lo and B tiles, and every B fragment feeds two MFMAs (three stages).
// K64: 64-k tiles (128-byte LDS rows) in a shallower ring: 2 stages for
// 256 x 256 tiles, 3 for 128 x 256, 4 for 128 x 128.
template <int BM, int BN, bool LO = false, bool K64 = false>
struct Cfg {
  static constexpr int BK = K64 ? 64 : 32;  // k per tile
  static constexpr int ROWB = BK * 2;       // bytes per LDS row
  static constexpr int CPR = BK / 8;        // 16-byte chunks per row
  // wave tile: 128 x 64 (256 x 256), 64 x 96 (256 x 192), else 64 x 64
  static constexpr int WM = BM == 256 && BN == 256 ? 128 : 64;
  static constexpr int WN = BN == 192 ? 96 : 64;
  static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
  static constexpr int NW = WAVES_M * WAVES_N;
  static constexpr int NT = 64 * NW;
  static constexpr int FM = WM / 32, FN = WN / 32;
  static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
  static constexpr int PARTS = LO ? 2 : 1;  // parts of A in a stage
  static constexpr int STAGE_BYTES = PARTS * A_BYTES + B_BYTES;
  static constexpr int A_LOADS = A_BYTES / (NT * 16), B_LOADS = B_BYTES / (NT * 16);  // per thread per k-tile
  static constexpr int LOADS = PARTS * A_LOADS + B_LOADS;
  static constexpr int ST = LO ? 3 : !K64 ? STAGES : (BM == 256 && BN >= 192) ? 2 : (BM * BN > 128 * 128) ? 3 : 4;
  static_assert(!(LO && K64), "the low part of A uses 32-k tiles");
  static constexpr int LDS_BYTES = ST * STAGE_BYTES;
  static_assert(A_LOADS >= 1 && B_LOADS >= 1 && A_BYTES % (NT * 16) == 0 && B_BYTES % (NT * 16) == 0, "tile split");
};

// Inputs that the epilogue of 8 consecutive output columns of one row reads
// from memory (the residual or the GELU inputs as raw bits, the row's
// exponent), loaded one 32-row strip ahead of their use so that their latency
// overlaps the staging of the previous strip.
struct EpiIn {
  u32x4 a, b;  // EPI_RESID: residual (bf16: a; fp32: a, b); EPI_DGELU: aux (a, b)
  int e;       // row exponent (EPI_RESID, EPI_GELU)
};

// Offset of output element (row, col) of shard column block nshard in the
// default output / residual layout: row * ldo + nshard * N_s + col.
__device__ __forceinline__ int64_t epi_index(const GemmArgs& g, int nshard, int row, int col) {
  return (int64_t)row * g.ldo + (int64_t)nshard * g.N_s + col;
}

template <int EPI>
__device__ __forceinline__ void load_row8(const GemmArgs& g, int nshard, int row, int col, EpiIn& in) {
  if constexpr (EPI == EPI_RESID) {
    in.e = g.row_exp ? g.row_exp[row] : 0;
    if (g.residual) {
      const int64_t idx = epi_index(g, nshard, row, col);
      if (g.res_f32) {
        const float* rp = static_cast<const float*>(g.residual) + idx;
        in.a = *reinterpret_cast<const u32x4*>(rp);
        in.b = *reinterpret_cast<const u32x4*>(rp + 4);
      } else {
        in.a = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(g.residual) + idx);
      }
    }
  } else if constexpr (EPI == EPI_DGELU) {
    const float* up = g.aux + (int64_t)row * g.N_s + col;
    in.a = *reinterpret_cast<const u32x4*>(up);
    in.b = *reinterpret_cast<const u32x4*>(up + 4);
  } else if constexpr (EPI == EPI_GELU) {
    in.e = g.row_exp ? g.row_exp[row] : 0;
  }
}

// Epilogue of 8 consecutive output columns of one row (fp32 values v[0..7],
// inputs `in` from load_row8): GELU (stored as fp16 scaled by 2^-row_exp) /
// row rescale and residual / Q-K-V routing, then 16-byte stores.  `col` is the
// column inside the shard's N_s block and a multiple of 8, so the 8 values
// never straddle a head or a Q/K/V part (head_dim is a multiple of 32).
template <int EPI>
__device__ __forceinline__ void store_row8(const GemmArgs& g, int nshard, int row, int col, float* v,
                                           const EpiIn& in) {
  u32x4 packed;
  if constexpr (EPI == EPI_RESID) {  // N-sharded: shard nshard writes column block nshard of the output
    const int64_t idx = epi_index(g, nshard, row, col);
    void* outp = g.out;  // separate output buffers per shard or per row block
    int64_t oidx = idx;
    if (g.outs[0]) {
      if (g.rows_per_out > 0) {
        const int k = row / g.rows_per_out;
        outp = g.outs[k];
        oidx = (int64_t)(row - k * g.rows_per_out) * g.ldo + col;
      } else {
        outp = g.outs[nshard];
        oidx = (int64_t)row * g.ldo + col;
      }
    }
    if (g.row_exp) {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = __builtin_amdgcn_ldexpf(v[j], in.e);
    }
    if (g.residual) {
      if (g.res_f32) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[j] += __uint_as_float(in.a[j]);
          v[4 + j] += __uint_as_float(in.b[j]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[2 * j] += __uint_as_float(in.a[j] << 16);
          v[2 * j + 1] += __uint_as_float(in.a[j] & 0xffff0000u);
        }
      }
    }
    if (g.out_f32) {
      float* op = static_cast<float*>(outp) + oidx;
      *reinterpret_cast<f32x4*>(op) = f32x4{v[0], v[1], v[2], v[3]};
      *reinterpret_cast<f32x4*>(op + 4) = f32x4{v[4], v[5], v[6], v[7]};
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) packed[j] = pack_bf16x2(v[2 * j], v[2 * j + 1]);
      *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(outp) + oidx) = packed;
    }
  } else if constexpr (EPI == EPI_DGELU) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] *= gelu_tanh_grad(__uint_as_float(in.a[j]));
      v[4 + j] *= gelu_tanh_grad(__uint_as_float(in.b[j]));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) packed[j] = pack_bf16x2(v[2 * j], v[2 * j + 1]);
    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(g.out) + epi_index(g, nshard, row, col)) = packed;
  } else if constexpr (EPI == EPI_GELU) {
    const int e = in.e;
    const int e_in = g.gelu_in_scaled ? e : 0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      packed[j] = pack_f16x2_sat(__builtin_amdgcn_ldexpf(gelu_tanh(__builtin_amdgcn_ldexpf(v[2 * j], e_in)), -e),
                                 __builtin_amdgcn_ldexpf(gelu_tanh(__builtin_amdgcn_ldexpf(v[2 * j + 1], e_in)), -e));
    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(g.out) + epi_index(g, nshard, row, col)) = packed;
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) packed[j] = pack_bf16x2(v[2 * j], v[2 * j + 1]);
    // columns of a shard: [Q heads | K heads | V heads], K and V possibly fewer
    const int hs_hd = g.heads_per_shard * g.head_dim;
    const int kv_hd = (g.kv_heads_per_shard ? g.kv_heads_per_shard : g.heads_per_shard) * g.head_dim;
    const int shard = nshard + g.shard0;
    if (col < hs_hd) {
      *reinterpret_cast<u32x4*>(g.q_out + (int64_t)row * g.hidden + shard * hs_hd + col) = packed;
    } else {
      const int is_v = col >= hs_hd + kv_hd;
      const int kcol = shard * kv_hd + (col - hs_hd - is_v * kv_hd);
      const int64_t gpos = row < g.chunk_len ? g.chunk_start0 + row : g.chunk_start1 + (row - g.chunk_len);
      uint16_t* dst = is_v ? g.v_full : g.k_full;
      *reinterpret_cast<u32x4*>(dst + gpos * (g.kv_ld ? g.kv_ld : g.hidden) + kcol) = packed;
    }
  }
}

template <int BM, int BN, int EPI, bool F16, bool LO = false, bool K64 = false>
__global__ __launch_bounds__((Cfg<BM, BN, LO, K64>::NT)) void gemm_kernel(const GemmArgs g) {
  using C = Cfg<BM, BN, LO, K64>;
  constexpr int BK = C::BK;
  // the LDS ring, then one word for the shard-arrival broadcast (a second
  // __shared__ object would make the compiler order every fragment read
  // behind all LDS-bound loads in flight)
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::LDS_BYTES + 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;

  const int tiles_m = (g.M + BM - 1) / BM;
  const int tiles_n_shard = (g.N_s + BN - 1) / BN;
  const int tiles_n = tiles_n_shard * g.n_shards;
  const int nwg = gridDim.x;
  int pid = blockIdx.x;
  if ((nwg & 7) == 0) pid = (pid & 7) * (nwg >> 3) + (pid >> 3);
  // tile rows per raster group: 8 for the QKV projection, 4 for the others
  // (measured: 4 rows help the W1, W2 and O GEMMs by 1-2 % and cost QKV 2 %)
  constexpr int GROUP_M = EPI == EPI_QKV ? 8 : 4;
  const int group_size = GROUP_M * tiles_n;
  const int first_m = (pid / group_size) * GROUP_M;
  const int gm = min(tiles_m - first_m, GROUP_M);
  const int in_group = pid % group_size;
  const int tm = first_m + in_group % gm;
  const int tn = in_group / gm;
  // column block in the raster order; with an arrival counter the N-sharded
  // blocks are taken in ring order from ring_start, so that each XCD's first
  // rounds of tiles need only the first shards to arrive
  const int nblock = tn / tiles_n_shard;
  const int nshard = g.arrived && g.k_shards == 1 ? (nblock + g.ring_start) % g.n_shards : nblock;
  const int n0 = (tn - nblock * tiles_n_shard) * BN;
  const int m0 = tm * BM;

  const int kt_per_shard = g.K_s / BK;
  const int reps = !LO && g.A_lo ? 2 : 1;  // K range of a shard walked once per part of A
  const int kt_per_rep = kt_per_shard * reps;
  const int k_tiles = kt_per_rep * g.k_shards;

  // ---- direct buffer->LDS loads.  Instruction i of wave w fills the 1 KB
  // block (i*NW + w) of the A (or B) region: 16 rows of 64 bytes; lane L ->
  // row L/4 of the block, physical chunk L%4 = logical chunk (L%4) ^
  // ((row/4)%4).  The byte offsets are relative to the tile's first row at
  // the k-tile's first column (the descriptors' base, rebased per k-tile in
  // SGPRs); rows past the matrix re-read its last row.
  // chunk swizzle: 64-byte rows c ^ ((r/4) % 4), 128-byte rows c ^ ((r/2) % 8)
  auto swz = [](int r) __attribute__((always_inline)) { return K64 ? ((r >> 1) & 7) : ((r >> 2) & 3); };
  constexpr int RPB = 1024 / C::ROWB;  // rows per 1 KB block
  uint32_t a_off[C::A_LOADS];
#pragma unroll
  for (int i = 0; i < C::A_LOADS; ++i) {
    const int r = (i * C::NW + wave) * RPB + lane / C::CPR;
    const int c = (lane % C::CPR) ^ swz(r);
    a_off[i] = (uint32_t)(((int64_t)(min(m0 + r, g.M - 1) - m0) * g.lda + c * 8) * 2);
  }
  uint32_t b_off[C::B_LOADS];
#pragma unroll
  for (int i = 0; i < C::B_LOADS; ++i) {
    const int r = (i * C::NW + wave) * RPB + lane / C::CPR;
    const int c = (lane % C::CPR) ^ swz(r);
    b_off[i] = (uint32_t)(((int64_t)(min(n0 + r, g.N_s - 1) - n0) * g.K_s + c * 8) * 2);
  }
  // bytes a descriptor covers: the tile's rows (the launch checks that they
  // fit in 2^31)
  const uint32_t a_bytes = (uint32_t)((int64_t)BM * g.lda * 2);
  const uint32_t b_bytes = (uint32_t)((int64_t)BN * g.K_s * 2);

  // Tiles are issued in order t = 0, 1, ...; the position of the next one
  // (k-tile within the shard, part of A, shard step of the ring) is walked
  // incrementally (wave-uniform scalars, no divisions).
  int nx_kt = 0, nx_part = 0, nx_d = g.k_shards > 1 ? g.ring_start : nshard;
  // Shard arrival: ring position of the next tile's shard, and the positions
  // known to have arrived (workgroup-uniform; INT32_MAX without a counter).
  uint32_t* const arrival_word = reinterpret_cast<uint32_t*>(smem + C::LDS_BYTES);
  int32_t avail = INT32_MAX, nx_pos = 0;
  if (g.arrived) {
    avail = -1;
    nx_pos = g.k_shards > 1 ? 0 : (nshard - g.ring_start + g.n_shards) % g.n_shards;
  }
  // Called by all waves alike: wave 0 polls until position `pos` has arrived
  // (or the poll budget is spent), then the count seen is passed to every
  // wave through LDS between two barriers, so all waves take the same
  // branches afterwards.  The poll is a system-scope load (past both cache
  // levels) and no acquire fence follows it: the shard's loads are issued
  // only after the poll's value has returned and the barriers have passed,
  // and nothing in this launch reads a shard before its arrival, so no line
  // of it is cached by this launch; lines left by earlier kernels (the
  // tests fill the shard buffers with NaN first) read fresh after arrival.
  // An agent-scope acquire here would invalidate the L2 under every other
  // tile of the XCD.
  auto await_arrival = [&](int32_t pos) __attribute__((always_inline)) -> int32_t {
    if (wave == 0) {
      typedef __attribute__((address_space(1))) uint32_t gu32;  // global, not flat: vm counter only
      const gu32* counter = (const gu32*)g.arrived;
      uint32_t seen = 0x7fffffffu;
      for (uint32_t k = 0;; ++k) {
        const uint32_t c = __hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) - g.arrived_base;
        if ((int32_t)c > pos) {
          seen = c;
          break;
        }
        if (k >= g.spin_limit) {
          if (lane == 0)
            __hip_atomic_store((gu32*)g.arrival_status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
          break;
        }
        __builtin_amdgcn_s_sleep(32);
      }
      if (lane == 0) *arrival_word = seen;
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the LDS write is done
    lds_barrier();
    const int32_t a = (int32_t)__builtin_amdgcn_readfirstlane(*arrival_word);
    lds_barrier();  // every wave has read the word before it can change
    return a;
  };
  // The matrices' pointers are kernel arguments; the current shard's weight
  // pointer is read again only at shard boundaries, and that scalar load is
  // waited for at once: a scalar load in flight shares the lgkm counter with
  // the fragment reads and would make the compiler wait for all of them.
  const uint16_t* a_hi = g.A + (int64_t)m0 * g.lda;
  const uint16_t* a_lo = g.A_lo + (int64_t)m0 * g.lda;
  const uint16_t* bshard = g.B[nx_d] + (int64_t)n0 * g.K_s;
  asm volatile("" ::"s"(a_hi), "s"(a_lo), "s"(bshard));  // in registers before the loop
  // Descriptors of the current shard's K range (A at the shard's first
  // column), rebuilt only at shard boundaries; a k-tile's column is the loads'
  // scalar offset, the same number of bytes into A and into B.
  __amdgpu_buffer_rsrc_t ra_hi, ra_lo, rb;
  auto shard_rsrc = [&]() __attribute__((always_inline)) {
    const int64_t acol = g.k_shards > 1 ? (int64_t)nx_d * g.K_s : 0;
    ra_hi = buffer_rsrc(a_hi + acol, a_bytes);
    ra_lo = buffer_rsrc(a_lo + acol, a_bytes);
    rb = buffer_rsrc(bshard, b_bytes);
  };
  shard_rsrc();
  auto issue_tile = [&](int t) __attribute__((always_inline)) {
    if (nx_pos >= avail) avail = await_arrival(nx_pos);
    const uint32_t soff = (uint32_t)nx_kt * (BK * 2);
    const __amdgpu_buffer_rsrc_t ra = nx_part ? ra_lo : ra_hi;
    const __amdgpu_buffer_rsrc_t rbt = rb;
    uint8_t* stage = smem + (t % C::ST) * C::STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < C::A_LOADS; ++i) dma16_buf(ra, a_off[i], stage + (i * C::NW + wave) * 1024, soff);
    if constexpr (LO) {
#pragma unroll
      for (int i = 0; i < C::A_LOADS; ++i)
        dma16_buf(ra_lo, a_off[i], stage + C::A_BYTES + (i * C::NW + wave) * 1024, soff);
    }
#pragma unroll
    for (int i = 0; i < C::B_LOADS; ++i)
      dma16_buf(rbt, b_off[i], stage + C::PARTS * C::A_BYTES + (i * C::NW + wave) * 1024, soff);
    if (++nx_kt == kt_per_shard) {
      nx_kt = 0;
      if (++nx_part == reps) {
        nx_part = 0;
        if (g.k_shards > 1) {
          if (++nx_d == g.k_shards) nx_d = 0;
          ++nx_pos;
          bshard = g.B[nx_d] + (int64_t)n0 * g.K_s;
          __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
          shard_rsrc();
        }
      }
    }
  };

  f32x16 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc[i][j] = f32x16{};

  // ---- fragment reads: row r = (wave rows) + 32*i + lane%32, logical chunk
  // 2*kk + lane/32, physical chunk (2*kk + lane/32) ^ ((r/4) % 4); the wave
  // row offsets are multiples of 32, so (r/4) % 4 = ((lane%32)/4) % 4.
  const int ql = lane & 31;
  const uint32_t xr = (uint32_t)(((lane >> 5) ^ swz(ql)) << 4);
  const uint32_t a_row = (uint32_t)(wm * C::WM + ql) * C::ROWB;
  const uint32_t b_row = (uint32_t)(C::PARTS * C::A_BYTES) + (uint32_t)(wn * C::WN + ql) * C::ROWB;

  // Both k-steps' fragments are read before the first step's MFMAs (step 0's
  // first), so each MFMA waits only for its own fragments.
  auto compute_tile = [&](int t) __attribute__((always_inline)) {
    const uint8_t* stage = smem + (t % C::ST) * C::STAGE_BYTES;
    u32x4 af[BK / 16][C::FM], bfv[BK / 16][C::FN];
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const uint32_t kx = xr ^ (uint32_t)(kk << 5);
#pragma unroll
      for (int i = 0; i < C::FM; ++i) af[kk][i] = *reinterpret_cast<const u32x4*>(stage + a_row + i * 32 * C::ROWB + kx);
#pragma unroll
      for (int j = 0; j < C::FN; ++j) bfv[kk][j] = *reinterpret_cast<const u32x4*>(stage + b_row + j * 32 * C::ROWB + kx);
      if constexpr (!LO) __builtin_amdgcn_sched_barrier(0);  // step 0's reads first
    }
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk)
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) acc[i][j] = mfma32_bits<F16>(af[kk][i], bfv[kk][j], acc[i][j]);
    if constexpr (!LO) {
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) __builtin_amdgcn_sched_group_barrier(0x008, C::FM * C::FN, 0);
    }
    if constexpr (LO) {  // the low part of A against the same B fragments
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        const uint32_t kx = xr ^ (uint32_t)(kk << 5);
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
          af[kk][i] = *reinterpret_cast<const u32x4*>(stage + C::A_BYTES + a_row + i * 32 * C::ROWB + kx);
      }
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk)
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
          for (int j = 0; j < C::FN; ++j) acc[i][j] = mfma32_bits<F16>(af[kk][i], bfv[kk][j], acc[i][j]);
    }
  };

  // ---- main loop: wait for tile t (the up to ST-2 tiles issued after it may
  // still be in flight), barrier (tile t visible to all waves; everyone is
  // done with tile t-1), compute tile t, then refill the stage of tile t-1
  // with tile t+ST-1; with two stages that refill (tile t+1) goes before the
  // MFMAs, so that it has the whole of tile t's compute to land.
  const int pro = min(C::ST - 1, k_tiles);
  for (int t = 0; t < pro; ++t) issue_tile(t);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // no scalar load in flight in the loop
  for (int t = 0; t < k_tiles; ++t) {
    const int ahead = min(k_tiles - 1 - t, C::ST - 2);  // tiles issued after t
    if (ahead >= 2)
      wait_vmcnt<2 * C::LOADS>();
    else if (ahead == 1)
      wait_vmcnt<C::LOADS>();
    else
      wait_vmcnt<0>();
    lds_barrier();
    if constexpr (C::ST == 2) {  // refill the other stage before the MFMAs
      if (t + 1 < k_tiles) issue_tile(t + 1);
      compute_tile(t);
    } else {
      compute_tile(t);
      if (t + C::ST - 1 < k_tiles) issue_tile(t + C::ST - 1);
    }
  }
  wait_vmcnt<0>();
  __syncthreads();

  // Epilogue, staged through LDS (free after the barrier above) so that global
  // stores are 16-byte row segments.  The 32x32 accumulator layout: lane holds
  // column (lane % 32) and rows 8*(e/4) + 4*(lane/32) + e%4 of its 16 values e.
  // Each wave stages one 32-row strip of its sub-tile at a time in fp32
  // ([32][WN + 4] floats), then reads it back as 8-column row pieces.  The
  // memory inputs of a strip's pieces (residual, GELU inputs, row exponents)
  // are loaded while the previous strip is staged and stored, so each tile
  // waits for that latency once instead of once per piece.
  {
    constexpr int SLD = C::WN + 4;  // padded fp32 row
    float* stage = reinterpret_cast<float*>(smem) + wave * 32 * SLD;
    const int col_l = lane & 31;
    const int row_l = 4 * (lane >> 5);
    constexpr int PIECES = 32 * (C::WN / 8);  // 8-column pieces in a strip
    constexpr int PPL = PIECES / 64;          // pieces per lane
    auto piece_rc = [&](int i, int it, int& row, int& col, int& r, int& c8) __attribute__((always_inline)) {
      const int piece = it * 64 + lane;
      r = piece / (C::WN / 8);
      c8 = (piece - r * (C::WN / 8)) * 8;
      row = m0 + wm * C::WM + i * 32 + r;
      col = n0 + wn * C::WN + c8;
    };
    EpiIn in[2][PPL];
    auto load_strip = [&](int i, EpiIn (&dst)[PPL]) __attribute__((always_inline)) {
#pragma unroll
      for (int it = 0; it < PPL; ++it) {
        int row, col, r, c8;
        piece_rc(i, it, row, col, r, c8);
        if (row < g.M && col < g.N_s) load_row8<EPI>(g, nshard, row, col, dst[it]);
      }
    };
    load_strip(0, in[0]);
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
      if (i + 1 < C::FM) load_strip(i + 1, in[(i + 1) & 1]);
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          stage[(8 * (e >> 2) + row_l + (e & 3)) * SLD + j * 32 + col_l] = acc[i][j][e];
      __syncthreads();
#pragma unroll
      for (int it = 0; it < PPL; ++it) {
        int row, col, r, c8;
        piece_rc(i, it, row, col, r, c8);
        float v[8];
        const f32x4 lo = *reinterpret_cast<const f32x4*>(stage + r * SLD + c8);
        const f32x4 hi = *reinterpret_cast<const f32x4*>(stage + r * SLD + c8 + 4);
#pragma unroll
        for (int k = 0; k < 4; ++k) { v[k] = lo[k]; v[4 + k] = hi[k]; }
        if (row < g.M && col < g.N_s) store_row8<EPI>(g, nshard, row, col, v, in[i & 1][it]);
      }
      __syncthreads();
    }
  }
}

template <int BM, int BN, bool K64>
hipError_t launch_tiles_k(const GemmArgs& g, hipStream_t stream) {
  const int tiles_m = (g.M + BM - 1) / BM;
  const int tiles_n = ((g.N_s + BN - 1) / BN) * g.n_shards;
  const dim3 grid(tiles_m * tiles_n), block(Cfg<BM, BN>::NT);
  // Instantiated: QKV (bf16), W1 + GELU (bf16 or fp16), O projection (bf16), W2 (fp16),
  // GELU-derivative product (bf16, MLP backward).
  switch (g.epilogue) {
    case EPI_QKV: hipLaunchKernelGGL((gemm_kernel<BM, BN, EPI_QKV, false, false, K64>), grid, block, 0, stream, g); break;
    case EPI_DGELU: hipLaunchKernelGGL((gemm_kernel<BM, BN, EPI_DGELU, false, false, K64>), grid, block, 0, stream, g); break;
    case EPI_GELU:
      if (g.f16)
        hipLaunchKernelGGL((gemm_kernel<BM, BN, EPI_GELU, true, false, K64>), grid, block, 0, stream, g);
      else
        hipLaunchKernelGGL((gemm_kernel<BM, BN, EPI_GELU, false, false, K64>), grid, block, 0, stream, g);
      break;
    default:
      if (g.f16)
        hipLaunchKernelGGL((gemm_kernel<BM, BN, EPI_RESID, true, false, K64>), grid, block, 0, stream, g);
      else if (g.A_lo)  // O projection on the attention output's two parts
        hipLaunchKernelGGL((gemm_kernel<BM, BN, EPI_RESID, false, true, false>), grid, block, 0, stream, g);
      else
        hipLaunchKernelGGL((gemm_kernel<BM, BN, EPI_RESID, false, false, K64>), grid, block, 0, stream, g);
      break;
  }
  return hipGetLastError();
}

template <int BM, int BN>
hipError_t launch_tiles(const GemmArgs& g, hipStream_t stream) {
  if (GEMM_K64 && g.K_s % 64 == 0 && !g.A_lo) return launch_tiles_k<BM, BN, true>(g, stream);
  return launch_tiles_k<BM, BN, false>(g, stream);
}

// The QKV projection on 256 x 192 tiles of 64-k (eight waves of 64 x 96), for
// shard widths that are multiples of 192.
hipError_t launch_qkv192(const GemmArgs& g, hipStream_t stream) {
  const dim3 grid(((g.M + 255) / 256) * (g.N_s / 192) * g.n_shards), block(Cfg<256, 192, false, true>::NT);
  hipLaunchKernelGGL((gemm_kernel<256, 192, EPI_QKV, false, false, true>), grid, block, 0, stream, g);
  return hipGetLastError();
}

// Compute units of the current device (queried once; 256 if the query fails).
int cu_count() {
  static int n = 0;
  if (n == 0) {
    int dev = 0, v = 0;
    const bool ok = hipGetDevice(&dev) == hipSuccess &&
                    hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess;
    n = ok && v > 0 ? v : 256;
  }
  return n;
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& g, hipStream_t stream) {
  if (g.M <= 0) return hipSuccess;
  // a tile's rows must fit one buffer descriptor (32-bit byte offsets)
  if ((int64_t)256 * g.lda * 2 > INT32_MAX || (int64_t)256 * g.K_s * 2 > INT32_MAX) return hipErrorInvalidValue;
  // 256 x 256 tiles keep the LDS traffic per MFMA low; fall back to 128 x 128
  // when the big tiles would leave most of the 256 CUs idle.
  const long big = (long)((g.M + 255) / 256) * (((g.N_s + 255) / 256) * g.n_shards);
  if (big >= 192) {
    // The QKV projection's shards are multiples of 192 wide: 256 x 192 tiles
    // when they fill the rounds of tiles on the CUs better.  A round of them
    // takes about 0.9 of a round of 256 x 256 tiles (measured at 2048 tokens,
    // for 0.75 of the work: lower operand reuse), e.g. 2048 tokens: 384 tiles
    // of 256 x 256 (1.5 rounds, so 2) or 512 of 256 x 192 (2 rounds, 1.8).
    if (g.epilogue == EPI_QKV && g.N_s % 192 == 0 && GEMM_K64 && g.K_s % 64 == 0 && !g.A_lo) {
      const long cu = cu_count();
      const long t192 = (long)((g.M + 255) / 256) * ((g.N_s / 192) * g.n_shards);
      const double r256 = (double)((big + cu - 1) / cu), r192 = 0.9 * (double)((t192 + cu - 1) / cu);
      if (r192 < r256) return launch_qkv192(g, stream);
    }
    return launch_tiles<256, 256>(g, stream);
  }
  // short token counts: 128 x 256 tiles (eight waves, 1.33x the bytes per flop
  // of 256 x 256) while they still fill the CUs, then 128 x 128
  const long mid = (long)((g.M + 127) / 128) * (((g.N_s + 255) / 256) * g.n_shards);
  if (mid >= 192 && g.N_s >= 256) return launch_tiles<128, 256>(g, stream);
  return launch_tiles<128, 128>(g, stream);
}

}  // namespace tsp
