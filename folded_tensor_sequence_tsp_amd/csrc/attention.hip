// Causal flash attention of a rank's two zigzag query chunks against the whole
// gathered K/V, for gfx950 (CDNA4).
//
// TSP gathers K/V over a zigzag partition of the sequence so that every rank
// holds one early and one late chunk of queries and the same causal work
// (zubnet.ai, "Zyphra TSP folds TP+SP onto one GPU axis", para. 2).  Here the
// queries of chunk i sit at global positions chunk_start[i] + row; a query at
// position p attends to keys 0..p of the full sequence.
//
// Design (one workgroup = one head x QT = 256 queries of one chunk, 8 waves of
// 32 queries, two waves per SIMD):
//   * scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//     each lane then holds ONE query (lane % 32) and 16 keys per 32-key block,
//     so the row max needs a single exchange with lane ^ 32 and row sums stay
//     per lane until the end;
//   * O^T = V^T P^T takes the probabilities from the score registers as the B
//     operand.  V is first rewritten per head as V^T tiles [64-key tile][d][64]
//     with the keys of each 16-key group in the order the score registers hold
//     them (vt_prep_kernel), so every lane's 8 keys of a k-step are one 16-byte
//     LDS read;
//   * K and V^T tiles of 64 keys stream into a 4-stage LDS ring with direct
//     global->LDS loads (global_load_lds_dwordx4; no register staging), the 16-
//     byte chunks of each row XOR-swizzled by the row index so that fragment
//     reads of 32 rows hit distinct banks of the 64-bank LDS; per tile one
//     vmcnt wait and one barrier; loads run two to three tiles ahead;
//   * software pipeline: the S MFMAs of tile t+1 sit in one basic block with
//     the exponentials of tile t (all branches are wave-uniform), so matrix
//     and vector work interleave; the PV MFMAs of tile t then overlap the max
//     of tile t+1's unmasked scores and the running sum of tile t (kept in that
//     block); a tile that crosses a wave's diagonal is masked after the block
//     and its max taken again;
//   * online softmax in fp32, log2 domain, scale folded into one FMA, hardware
//     exp2, and lazy rescaling: the running max moves (and O, l are rescaled)
//     only when a tile's max exceeds it by more than 2^8, so probabilities stay
//     below 256 and most tiles skip the rescale;
//   * masking only on tiles that cross a wave's diagonal; tiles past a wave's
//     last query are not computed;
//   * grouped-query attention: query head a reads K/V head a / (H / H_kv); the
//     query heads of one K/V head are neighbours in the workgroup order, so
//     they meet its K/V in the same XCD's L2;
//   * workgroups ordered so each XCD works through a contiguous range of heads,
//     heaviest (latest) query tiles first;
//   * when the grid is small (few query tiles: short sequences), the late
//     chunk's tiles, which see almost the whole sequence while the early
//     chunk's see a few tiles, are split in two along the keys: each half
//     writes its unnormalised output with its running max and sum, and a
//     combine kernel merges the halves (the same algebra as the lazy rescale).
#include "device_common.h"
#include "kernels.h"

namespace tsp {
namespace {

constexpr int NW = 8;              // waves per workgroup
constexpr int NTHREADS = 64 * NW;
constexpr int QT = 32 * NW;        // queries per workgroup
constexpr int BKV = 64;            // keys per tile
constexpr int NSTAGE = 4;          // LDS ring depth
constexpr float LAZY_TAU = 8.0f;   // rescale threshold (log2 units)

template <int HD>
struct ACfg {
  static constexpr int NCH = HD / 8;              // 16-byte chunks per K row
  static constexpr int K_BYTES = BKV * HD * 2;    // K tile [64][HD]
  static constexpr int V_BYTES = HD * BKV * 2;    // V^T tile [HD][64]
  static constexpr int STAGE_BYTES = K_BYTES + V_BYTES;
  static constexpr int K_LOADS = K_BYTES / (NTHREADS * 16);  // DMA instructions per thread per tile
  static constexpr int V_LOADS = V_BYTES / (NTHREADS * 16);
  static constexpr int LOADS = K_LOADS + V_LOADS;
  static constexpr int K_ROWS_PER_LOAD = 64 / NCH;            // K rows one wave instruction fills
  static constexpr int KK = HD / 16;                          // MFMA k-steps over head_dim
  static constexpr int DT = HD / 32;                          // 32-wide d tiles of O
  static_assert(K_LOADS >= 1 && V_LOADS >= 1, "tile too small for the workgroup");
};

// Position k (0..15) of a 16-key group of V^T holds key perm(k): bits 2 and 3
// swapped.  A lane of half h holds in its score registers the keys
// {4h..4h+3, 8+4h..8+4h+3} of each 16-key group, i.e. perm(8h + j), j = 0..7.
__device__ __forceinline__ int key_perm16(int k) { return (k & 3) | ((k & 4) << 1) | ((k & 8) >> 1); }

// V [S x ld] (head columns head*HD .. +HD-1) -> V^T tiles
// vt[((head * n_kv_tiles + t) * HD + d) * 64 + k] = V[t*64 + key_perm16-order(k)][head*HD + d], 0 past S.
// One thread moves 8 keys x 8 dims: eight 16-byte row reads, an 8x8 transpose
// in registers, eight 16-byte writes (8 consecutive lanes write one 128-byte row).
template <int HD>
__global__ __launch_bounds__(128) void vt_prep_kernel(const uint16_t* __restrict__ v, int64_t S, int32_t ld,
                                                      uint16_t* __restrict__ vt, int64_t n_kv_tiles) {
  constexpr int NCH = HD / 8;
  const int t = blockIdx.x;
  const int head = blockIdx.y;
  for (int item = threadIdx.x; item < 8 * NCH; item += 128) {
    const int kg = item & 7;     // 8-slot group: slots 8*kg .. 8*kg+7 of the tile
    const int dc = item >> 3;    // dims 8*dc .. 8*dc+7
    uint32_t r[8][4];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int slot = 8 * kg + j;
      const int64_t key = (int64_t)t * 64 + (slot & ~15) + key_perm16(slot & 15);
      if (key < S) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(v + key * ld + head * HD + dc * 8);
        r[j][0] = x[0]; r[j][1] = x[1]; r[j][2] = x[2]; r[j][3] = x[3];
      } else {
        r[j][0] = r[j][1] = r[j][2] = r[j][3] = 0u;
      }
    }
    uint16_t* dst = vt + (((int64_t)head * n_kv_tiles + t) * HD + dc * 8) * 64 + 8 * kg;
#pragma unroll
    for (int i = 0; i < 8; ++i) {  // dim dc*8 + i: keys j = 0..7
      u32x4 w;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t a0 = (i & 1) ? (r[2 * m][i >> 1] >> 16) : (r[2 * m][i >> 1] & 0xffffu);
        const uint32_t a1 = (i & 1) ? (r[2 * m + 1][i >> 1] & 0xffff0000u) : (r[2 * m + 1][i >> 1] << 16);
        w[m] = a0 | a1;
      }
      *reinterpret_cast<u32x4*>(dst + i * 64) = w;
    }
  }
}

template <int HD, bool SPLIT>
__global__ __launch_bounds__(NTHREADS) void attn_kernel(const AttnArgs a) {
  using C = ACfg<HD>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NSTAGE * C::STAGE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar) index
  const int half = lane >> 5;
  const int ql = lane & 31;

  // ---- work item: (head, chunk, tile), heaviest tiles of a head first, heads
  // contiguous per XCD.  SPLIT: (head, chunk 1, tile, key half) items first,
  // then the chunk-0 tiles whole.
  const int tpc = (int)((a.chunk_len + QT - 1) / QT);
  const int per_head = (SPLIT ? 3 : 2) * tpc;
  const int nwg = gridDim.x;
  int pid = blockIdx.x;
  if ((nwg & 7) == 0) pid = (pid & 7) * (nwg >> 3) + (pid >> 3);
  const int head = pid / per_head;
  const int w = pid - head * per_head;
  const int n1 = SPLIT ? 2 * tpc : tpc;  // items of chunk 1
  const int chunk = w < n1 ? 1 : 0;
  const int tile = w < n1 ? tpc - 1 - (SPLIT ? w >> 1 : w) : per_head - 1 - w;
  const int part = SPLIT && chunk ? (w & 1) : -1;  // key half of a split item, -1: whole

  const int64_t row0 = (int64_t)chunk * a.chunk_len + (int64_t)tile * QT;  // local row of query 0
  const int64_t pos0 = (chunk ? a.chunk_start1 : a.chunk_start0) + (int64_t)tile * QT;
  const int valid = (int)min((int64_t)QT, a.chunk_len - (int64_t)tile * QT);
  const int64_t key_end = pos0 + valid;  // keys [0, key_end)
  const int n_tiles = (int)((key_end + BKV - 1) / BKV);
  // key tiles [t_begin, t_end) of this item; a split's first half ends before
  // the tile's first query, so only the second half crosses the diagonal
  int t_begin = 0, t_end = n_tiles;
  if (SPLIT && part >= 0) {
    const int mid = (int)min((int64_t)(n_tiles / 2), pos0 / BKV);
    if (part == 0)
      t_end = mid;
    else
      t_begin = mid;
  }

  // This lane's query (clamped to the last valid row for the ragged tail).
  const int qi = min(wave * 32 + ql, valid - 1);
  const int64_t qpos = pos0 + qi;
  const int wave_first = wave * 32;
  const bool wave_active = wave_first < valid;
  const int64_t wave_min_pos = pos0 + wave_first;
  const int64_t wave_max_pos = pos0 + min(wave_first + 31, valid - 1);
  const int wave_tiles = wave_active ? (int)(wave_max_pos / BKV) + 1 : 0;  // tiles 0..wave_tiles-1 computed

  const int hcol = head * HD;
  const int64_t ld = a.hidden;
  const int kvh = head / (a.n_heads / a.kv_heads);  // this head's K/V head
  const int kcol = kvh * HD;
  const int64_t kld = a.kv_ld;

  // ---- Q fragments in registers: lane holds query ql, dims kk*16 + 8*half .. +7.
  bf16x8 qf[C::KK];
  {
    const uint16_t* qp = a.q + (row0 + qi) * ld + hcol + 8 * half;
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) qf[kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(qp + kk * 16));
  }

  // ---- direct global->LDS loads.  Instruction i of wave w fills the 1 KB
  // block (i*NW + w) of a tile region; lane L writes its 16 bytes at L*16.
  // K: row r of the tile, logical 16-byte chunk (L % NCH) ^ (r % NCH).
  int k_row[C::K_LOADS];             // K row (key within the tile) this lane fetches
  int k_col[C::K_LOADS];             // element column within the head (swizzled chunk)
  const uint16_t* k_src[C::K_LOADS];  // source for tile 0; tile t adds t * 64 rows
#pragma unroll
  for (int i = 0; i < C::K_LOADS; ++i) {
    const int r = (i * NW + wave) * C::K_ROWS_PER_LOAD + lane / C::NCH;
    const int p = lane % C::NCH;
    k_row[i] = r;
    k_col[i] = (p ^ (r & (C::NCH - 1))) * 8;
    k_src[i] = a.k + (int64_t)r * kld + kcol + k_col[i];
  }
  // V^T: row d of the tile, logical chunk (L % 8) ^ ((d / 2) % 8).
  const uint16_t* v_src[C::V_LOADS];
  {
    const uint16_t* vt_head = a.vt + (int64_t)kvh * a.n_kv_tiles * HD * 64;
#pragma unroll
    for (int i = 0; i < C::V_LOADS; ++i) {
      const int d = (i * NW + wave) * 8 + lane / 8;
      const int p = lane % 8;
      v_src[i] = vt_head + d * 64 + (p ^ ((d >> 1) & 7)) * 8;
    }
  }

  auto issue_tile = [&](int t) __attribute__((always_inline)) {
    uint8_t* stage = smem + (t % NSTAGE) * C::STAGE_BYTES;
    const int64_t k0 = (int64_t)t * BKV;
    if (k0 + BKV <= key_end) {  // whole tile inside the key range (wave-uniform)
#pragma unroll
      for (int i = 0; i < C::K_LOADS; ++i) dma16(k_src[i] + k0 * kld, stage + (i * NW + wave) * 1024);
    } else {                    // last tile: rows past the range re-read the last key (masked anyway)
#pragma unroll
      for (int i = 0; i < C::K_LOADS; ++i) {
        const int64_t key = min(k0 + k_row[i], key_end - 1);
        dma16(a.k + key * kld + kcol + k_col[i], stage + (i * NW + wave) * 1024);
      }
    }
#pragma unroll
    for (int i = 0; i < C::V_LOADS; ++i)
      dma16(v_src[i] + (int64_t)t * HD * 64, stage + C::K_BYTES + (i * NW + wave) * 1024);
  };

  // ---- fragment read addresses (bytes within a stage).  K row r = kb*32 + ql,
  // logical chunk 2*kk + half, physical chunk (2*kk + half) ^ (r % NCH):
  // address = (row base | ((half ^ r%NCH) << 4)) ^ (kk << 5).  V^T row
  // d = dt*32 + ql (128 bytes), chunk 2*ks + half, physical chunk
  // (2*ks + half) ^ ((d/2) % 8): with 64 LDS banks two consecutive rows cover
  // all banks, so 16 lanes (rows d..d+15) then hit distinct banks.
  const uint32_t k_a0 = (uint32_t)ql * (HD * 2) + ((uint32_t)(half ^ (ql & (C::NCH - 1))) << 4);
  const uint32_t v_a0 = C::K_BYTES + (uint32_t)ql * 128 + ((uint32_t)(half ^ ((ql >> 1) & 7)) << 4);

  // S^T for tile t: lane holds query ql, keys 8*(e/4) + 4*half + e%4 of each 32-key block.
  auto compute_s = [&](int t, f32x16 (&s)[2]) __attribute__((always_inline)) {
    const uint8_t* stage = smem + (t % NSTAGE) * C::STAGE_BYTES;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < C::KK; ++kk) {
        const u32x4 kf = *reinterpret_cast<const u32x4*>(stage + kb * 32 * (HD * 2) + (k_a0 ^ (uint32_t)(kk << 5)));
        s[kb] = mfma32(as_bf16x8(kf), qf[kk], s[kb]);
      }
    }
  };

  // ---- running state (log2 domain): m = running reference max of the scaled
  // scores, l = lane-partial sum of exp2(score*scale - m).
  constexpr float inv_sqrt_hd = HD == 128 ? 0.08838834764831844055f : 0.125f;
  const float scale_log2 = 1.44269504088896340736f * inv_sqrt_hd;
  float m_run = -INFINITY;
  float l_run = 0.0f;
  f32x16 o[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) o[dt] = f32x16{};

  // Causal mask of tile t's scores when the tile crosses the wave's diagonal.
  auto mask_tile = [&](int t, f32x16 (&s)[2]) __attribute__((always_inline)) {
    const int64_t k0 = (int64_t)t * BKV;
    if (k0 + BKV - 1 > wave_min_pos) {  // wave-uniform
      // key k0 + kb*32 + 8*(e/4) + 4*half + e%4 is masked when it exceeds qpos,
      // i.e. when the lane-independent part kb*32 + 8*(e/4) + e%4 exceeds lim.
      const int lim = (int)min(max(qpos - k0, (int64_t)-1), (int64_t)BKV) - 4 * half;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (kb * 32 + 8 * (e >> 2) + (e & 3) > lim) s[kb][e] = -INFINITY;
    }
  };

  // Scaled row max of a tile's (masked) scores, combined over the lane pair
  // (lanes l and l+32 hold the two halves of a query's keys).
  auto tile_max = [&](f32x16 (&s)[2]) __attribute__((always_inline)) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kb][e]);
    return pair_max(mx) * scale_log2;
  };

  // The fused block of a step: S of tile t+1 as two interleaved MFMA chains
  // (the two 32-key blocks) over the head_dim steps, with the K fragments of
  // the next step read before the current MFMAs and the exponentials of tile
  // t's keys 0..31 spread over the steps; then PV of tile t as DT independent
  // chains over the four 16-key steps, V^T fragments again one step ahead, the
  // exponentials of keys 32..63 under its first two steps and the max of tile
  // t+1's (unmasked) scores under the last two.  The vector work is
  // split so that each MFMA carries a few vector instructions (co-issued), and
  // LDS latency hides behind MFMAs.
  auto fused_block = [&](int t, f32x16 (&s_cu)[2], f32x16 (&s_nx)[2], float& mt) __attribute__((always_inline)) {
    const uint8_t* kst = smem + ((t + 1) % NSTAGE) * C::STAGE_BYTES;
    const uint8_t* vst = smem + (t % NSTAGE) * C::STAGE_BYTES;
    auto kfrag = [&](int kb, int kk) __attribute__((always_inline)) {
      return *reinterpret_cast<const u32x4*>(kst + kb * 32 * (HD * 2) + (k_a0 ^ (uint32_t)(kk << 5)));
    };
    auto vfrag = [&](int dt, int ks) __attribute__((always_inline)) {
      return *reinterpret_cast<const u32x4*>(vst + dt * 32 * 128 + (v_a0 ^ (uint32_t)(ks << 5)));
    };
    constexpr int PAIRS = 8 / C::KK;  // probability pairs of keys 0..31 per head_dim step
    const float neg_m = -m_run;
    float lsum = 0.0f;
    uint32_t pk[16];  // bf16 pairs: pk[4*ks + j] holds keys of 16-key step ks
    // probabilities of the score pair idx (keys 2*idx, 2*idx+1 of the lane's order)
    auto prob_pair = [&](int idx) __attribute__((always_inline)) {
      const int kb = idx >> 3, e = (2 * idx) & 15;
      const float p0 = __builtin_amdgcn_exp2f(fmaf(s_cu[kb][e], scale_log2, neg_m));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(s_cu[kb][e + 1], scale_log2, neg_m));
      lsum += p0 + p1;
      pk[idx] = pack_bf16x2(p0, p1);
    };
    u32x4 a0 = kfrag(0, 0), a1 = kfrag(1, 0);
    s_nx[0] = f32x16{};
    s_nx[1] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {
      u32x4 b0 = a0, b1 = a1;
      if (kk + 1 < C::KK) {
        b0 = kfrag(0, kk + 1);
        b1 = kfrag(1, kk + 1);
      }
      s_nx[0] = mfma32(as_bf16x8(a0), qf[kk], s_nx[0]);
      s_nx[1] = mfma32(as_bf16x8(a1), qf[kk], s_nx[1]);
#pragma unroll
      for (int q = 0; q < PAIRS; ++q) prob_pair(kk * PAIRS + q);  // keys 0..31
      a0 = b0;
      a1 = b1;
    }
    u32x4 v[C::DT];
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) v[dt] = vfrag(dt, 0);
    float mx = -INFINITY;  // max of tile t+1's unmasked scores, under the PV MFMAs
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 w[C::DT];
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) w[dt] = ks + 1 < 4 ? vfrag(dt, ks + 1) : v[dt];
      const bf16x8 p = as_bf16x8(u32x4{pk[4 * ks], pk[4 * ks + 1], pk[4 * ks + 2], pk[4 * ks + 3]});
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) o[dt] = mfma32(as_bf16x8(v[dt]), p, o[dt]);
      if (ks < 2) {  // keys 32..63, needed from step 2 on, under the MFMAs of steps 0 and 1
#pragma unroll
        for (int q = 0; q < 4; ++q) prob_pair(8 + 4 * ks + q);
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s_nx[ks - 2][e]);
      }
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) v[dt] = w[dt];
    }
    l_run += lsum;
    asm volatile("" : "+v"(l_run));  // keep the sum in this block, under the MFMAs
    mt = pair_max(mx) * scale_log2;
  };

  // One pipeline step: make tile t+1 visible (and the stage of tile t-1 free);
  // for tile t: the rare lazy rescale (a wave-uniform branch on the max mt of
  // tile t, found in the previous step), then the fused block (S of tile t+1,
  // exponentials and PV of tile t, then the mask and max of tile t+1 under the
  // PV MFMAs); last, issue the loads of tile t+NSTAGE-1 (issued after the
  // compute, the loads do not hold up the wave's MFMAs).
  auto step = [&](int t, f32x16 (&s_cu)[2], f32x16 (&s_nx)[2], float& mt, auto masked) __attribute__((always_inline)) {
    if (t + 1 < t_end) {
      if (t + 2 < t_end)
        wait_vmcnt<C::LOADS>();
      else
        wait_vmcnt<0>();
    }
    lds_barrier();
    if (t < wave_tiles) {  // wave-uniform
      if (__builtin_amdgcn_ballot_w64(mt > m_run + LAZY_TAU) != 0) {  // wave-uniform, rare
        const float m_new = fmaxf(m_run, mt);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) o[dt] *= alpha;
      }
      // S of tile t+1 is computed even past the wave's last tile (it then reads
      // a stale stage and is never used), keeping the block branch-free.
      fused_block(t, s_cu, s_nx, mt);
      // tile t+1 crosses the wave's diagonal (rare): mask it and take its max
      // again (the block's max is of the unmasked scores)
      if constexpr (decltype(masked)::value) {
        if ((int64_t)(t + 1) * BKV + BKV - 1 > wave_min_pos) {  // wave-uniform
          mask_tile(t + 1, s_nx);
          mt = tile_max(s_nx);
        }
      }
    }
    if (t + NSTAGE - 1 < t_end) issue_tile(t + NSTAGE - 1);
  };

  // ---- prologue: tiles t_begin .. t_begin+NSTAGE-2 in flight, wait for the first.
  const int pro = max(min(NSTAGE - 1, t_end - t_begin), 0);
  for (int t = t_begin; t < t_begin + pro; ++t) issue_tile(t);
  if (pro >= 3)
    wait_vmcnt<2 * C::LOADS>();
  else if (pro == 2)
    wait_vmcnt<C::LOADS>();
  else
    wait_vmcnt<0>();
  lds_barrier();

  f32x16 sA[2], sB[2];
  float mt = -INFINITY;  // scaled max of the current tile's masked scores
  if (t_begin < t_end && t_begin < wave_tiles) {
    compute_s(t_begin, sA);
    mask_tile(t_begin, sA);
    mt = tile_max(sA);
  }
  // Steps whose next tiles lie wholly at or before the workgroup's first
  // query carry no mask code (a wave-uniform branch there is if-converted by
  // the compiler into selects on every step); the rest, the diagonal tail,
  // mask.  Pairs keep the two score buffers' roles.
  const int t_m = (int)((pos0 + 1) / BKV);  // first tile that some wave masks
  int t = t_begin;
  for (; t + 1 < t_end && t + 2 < t_m; t += 2) {
    step(t, sA, sB, mt, std::false_type{});
    step(t + 1, sB, sA, mt, std::false_type{});
  }
  for (; t < t_end; t += 2) {
    step(t, sA, sB, mt, std::true_type{});
    if (t + 1 < t_end) step(t + 1, sB, sA, mt, std::true_type{});
  }
  wait_vmcnt<0>();

  if (SPLIT && part >= 0) {
    // unnormalised output, running max (log2 units) and sum of this key half
    if (wave_active && wave_first + ql < valid) {
      const float l_tot = l_run + __shfl_xor(l_run, 32);
      const int64_t r1 = (int64_t)tile * QT + wave_first + ql;  // row within chunk 1
      float* op = a.part_o + ((int64_t)part * a.chunk_len + r1) * ld + hcol + 4 * half;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<f32x4*>(op + dt * 32 + 8 * g) =
              f32x4{o[dt][4 * g], o[dt][4 * g + 1], o[dt][4 * g + 2], o[dt][4 * g + 3]};
      if (half == 0) {
        float* ml = a.part_ml + (((int64_t)part * a.n_heads + head) * a.chunk_len + r1) * 2;
        ml[0] = m_run;
        ml[1] = l_tot;
      }
    }
    return;
  }

  // ---- normalise and store: lane holds query ql, dims dt*32 + 8*(e/4) + 4*half + e%4.
  if (wave_active) {
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (a.lse && half == 0 && wave_first + ql < valid)  // sum_j exp(s_j) = 2^m_run * l_tot
      a.lse[(int64_t)head * 2 * a.chunk_len + row0 + wave_first + ql] =
          (m_run + log2f(l_tot)) * 0.69314718055994530942f;
    if (wave_first + ql < valid) {
      const float inv = 1.0f / l_tot;
      const int64_t off = (row0 + wave_first + ql) * ld + hcol + 4 * half;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float r[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) r[j] = o[dt][4 * g + j] * inv;
          u32x2 v;
          v[0] = pack_bf16x2(r[0], r[1]);
          v[1] = pack_bf16x2(r[2], r[3]);
          *reinterpret_cast<u32x2*>(a.o + off + dt * 32 + 8 * g) = v;
          if (a.o_lo) {  // rounding residual: r - bf16(r), itself rounded to bf16
            u32x2 wv;
            wv[0] = pack_bf16x2(r[0] - __uint_as_float(v[0] << 16), r[1] - __uint_as_float(v[0] & 0xffff0000u));
            wv[1] = pack_bf16x2(r[2] - __uint_as_float(v[1] << 16), r[3] - __uint_as_float(v[1] & 0xffff0000u));
            *reinterpret_cast<u32x2*>(a.o_lo + off + dt * 32 + 8 * g) = wv;
          }
        }
      }
    }
  }
}

// Merge the two key halves of the late chunk's rows: with (m_p, l_p, o_p) the
// running max (log2 units), sum and unnormalised output of half p and
// M = max(m_0, m_1), the row's output is
// (o_0 2^(m_0-M) + o_1 2^(m_1-M)) / (l_0 2^(m_0-M) + l_1 2^(m_1-M)).
// One thread per (row, head, 8 columns); an empty first half has m_0 = -inf.
template <int HD>
__global__ __launch_bounds__(256) void attn_combine_kernel(const AttnArgs a) {
  constexpr int G = HD / 8;  // 8-column groups per head
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = a.chunk_len * a.n_heads * G;
  if (idx >= total) return;
  const int g = (int)(idx % G);
  const int head = (int)((idx / G) % a.n_heads);
  const int64_t r1 = idx / ((int64_t)G * a.n_heads);
  const float* ml0 = a.part_ml + ((int64_t)head * a.chunk_len + r1) * 2;
  const float* ml1 = a.part_ml + (((int64_t)a.n_heads + head) * a.chunk_len + r1) * 2;
  const float m0 = ml0[0], l0 = ml0[1], m1 = ml1[0], l1 = ml1[1];
  const float M = fmaxf(m0, m1);
  const float w0 = __builtin_amdgcn_exp2f(m0 - M), w1 = __builtin_amdgcn_exp2f(m1 - M);
  const float L = l0 * w0 + l1 * w1;
  const float inv = 1.0f / L;
  const int64_t col = (int64_t)head * HD + 8 * g;
  const float* o0 = a.part_o + r1 * a.hidden + col;
  const float* o1 = a.part_o + (a.chunk_len + r1) * a.hidden + col;
  float r[8];
#pragma unroll
  for (int h4 = 0; h4 < 2; ++h4) {
    const f32x4 x0 = *reinterpret_cast<const f32x4*>(o0 + 4 * h4);
    const f32x4 x1 = *reinterpret_cast<const f32x4*>(o1 + 4 * h4);
#pragma unroll
    for (int j = 0; j < 4; ++j) r[4 * h4 + j] = (x0[j] * w0 + x1[j] * w1) * inv;
  }
  const int64_t off = (a.chunk_len + r1) * a.hidden + col;  // local row of chunk 1
  u32x4 v;
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = pack_bf16x2(r[2 * j], r[2 * j + 1]);
  *reinterpret_cast<u32x4*>(a.o + off) = v;
  if (a.o_lo) {
    u32x4 wv;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      wv[j] = pack_bf16x2(r[2 * j] - __uint_as_float(v[j] << 16), r[2 * j + 1] - __uint_as_float(v[j] & 0xffff0000u));
    *reinterpret_cast<u32x4*>(a.o_lo + off) = wv;
  }
  if (a.lse && g == 0) a.lse[(int64_t)head * 2 * a.chunk_len + a.chunk_len + r1] = (M + log2f(L)) * 0.69314718055994530942f;
}

constexpr int64_t SPLIT_BELOW = 512;  // split the late chunk's tiles when the grid has fewer items

bool attn_split(int64_t chunk_len, int32_t n_heads) {
  const int64_t tpc = (chunk_len + QT - 1) / QT;
  return chunk_len > 0 && 2 * (int64_t)n_heads * tpc < SPLIT_BELOW;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

int64_t attn_kv_tiles(int64_t seq_len) { return (seq_len + BKV - 1) / BKV; }

size_t attn_core_workspace(int64_t seq_len, int64_t chunk_len, int32_t hidden, int32_t n_heads) {
  size_t bytes = align256((size_t)attn_kv_tiles(seq_len) * 64 * hidden * 2);  // V^T tiles
  if (attn_split(chunk_len, n_heads))
    bytes += align256((size_t)2 * chunk_len * hidden * 4) + align256((size_t)2 * n_heads * chunk_len * 2 * 4);
  return bytes;
}

hipError_t launch_vt_tiles(const uint16_t* src, int64_t rows, int32_t ld, int32_t heads, int32_t head_dim,
                           uint16_t* dst, int64_t n_tiles, hipStream_t stream) {
  if (rows <= 0 || n_tiles <= 0) return hipSuccess;
  const dim3 grid((unsigned)n_tiles, (unsigned)heads), block(128);
  if (head_dim == 128)
    hipLaunchKernelGGL(vt_prep_kernel<128>, grid, block, 0, stream, src, rows, ld, dst, n_tiles);
  else
    hipLaunchKernelGGL(vt_prep_kernel<64>, grid, block, 0, stream, src, rows, ld, dst, n_tiles);
  return hipGetLastError();
}

hipError_t launch_vt_prep(const AttnArgs& a, hipStream_t stream) {
  return launch_vt_tiles(a.v, a.seq_len, a.kv_ld, a.kv_heads, a.head_dim, a.vt, a.n_kv_tiles, stream);
}

hipError_t launch_attention(const AttnArgs& args, hipStream_t stream) {
  if (args.chunk_len <= 0) return hipSuccess;
  hipError_t e = launch_vt_prep(args, stream);
  if (e != hipSuccess) return e;
  const int tpc = (int)((args.chunk_len + QT - 1) / QT);
  const dim3 block(NTHREADS);
  if (!attn_split(args.chunk_len, args.n_heads)) {
    const dim3 grid(args.n_heads * 2 * tpc);
    if (args.head_dim == 128)
      hipLaunchKernelGGL((attn_kernel<128, false>), grid, block, 0, stream, args);
    else
      hipLaunchKernelGGL((attn_kernel<64, false>), grid, block, 0, stream, args);
    return hipGetLastError();
  }
  // the key halves' partials follow the V^T tiles in the workspace
  AttnArgs a = args;
  char* base = reinterpret_cast<char*>(a.vt) + align256((size_t)a.n_kv_tiles * 64 * a.hidden * 2);
  a.part_o = reinterpret_cast<float*>(base);
  a.part_ml = reinterpret_cast<float*>(base + align256((size_t)2 * a.chunk_len * a.hidden * 4));
  const dim3 grid(a.n_heads * 3 * tpc);
  const unsigned cgrid = (unsigned)((a.chunk_len * a.n_heads * (a.head_dim / 8) + 255) / 256);
  if (a.head_dim == 128) {
    hipLaunchKernelGGL((attn_kernel<128, true>), grid, block, 0, stream, a);
    hipLaunchKernelGGL(attn_combine_kernel<128>, dim3(cgrid), dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL((attn_kernel<64, true>), grid, block, 0, stream, a);
    hipLaunchKernelGGL(attn_combine_kernel<64>, dim3(cgrid), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace tsp
