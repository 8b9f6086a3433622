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
//     operand.  V stays row-major (as gathered); its A-operand fragments come
//     from gfx950's transposing LDS reads (ds_read_b64_tr_b16), two per
//     fragment, with the keys of each 16-key group taken in the order the
//     score registers hold them;
//   * K and V tiles of 64 keys stream into a 4-stage LDS ring with direct
//     buffer->LDS loads (buffer_load_dwordx4 ... lds; no register staging).
//     The buffer descriptors are rebased per tile in SGPRs, so the per-lane
//     state is one 32-bit offset per load.  K rows are XOR-swizzled by the row
//     index (fragment reads of 32 rows hit distinct banks); V rows by the row
//     index mod 4 (the four rows of one transposing read fall in different
//     bank ranges).  Per tile one vmcnt wait and one barrier; loads run two to
//     three tiles ahead;
//   * software pipeline: the S MFMAs of tile t+1 sit in one basic block with
//     the exponentials of tile t (all branches are wave-uniform), so matrix
//     and vector work interleave; the PV MFMAs of tile t then overlap the max
//     of tile t+1's unmasked scores and the running sum of tile t (kept in that
//     block); a tile that crosses a wave's diagonal is masked after the block
//     and its max taken again;
//   * online softmax in fp32 with the hardware exp2 and lazy rescaling: the
//     running max moves (and O, l are rescaled) only when a tile's max exceeds
//     it by more than 2^8 after scaling, so probabilities stay below 256 and
//     most tiles skip the rescale.  The running max is kept in raw score units
//     and each exponent is (s - m) * log2(e)/sqrt(hd): the difference is exact
//     for the scores near the max at any magnitude, so the exponent of the
//     maximum is exactly 0 even when the scores are so large that their fp32
//     spacing exceeds the exponent range (activations of a deep stack without
//     a norm);
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
//
// The V^T tile pre-pass (vt_prep_kernel) is kept for the backward kernels,
// which stage K^T, Q^T and dO^T tiles at head_dim 64.
#include "device_common.h"
#include "kernels.h"

namespace tsp {
namespace {

constexpr int NW = 8;              // waves per workgroup
constexpr int NTHREADS = 64 * NW;
constexpr int QT = ATTN_QT;        // queries per workgroup (32 per wave)
constexpr int BKV = ATTN_BKV;      // keys per tile
constexpr int NSTAGE = 4;          // LDS ring depth
constexpr float LAZY_TAU = 8.0f;   // rescale threshold (log2 units)
static_assert(QT == 32 * NW, "one 32-query block per wave");

template <int HD>
struct ACfg {
  static constexpr int NCH = HD / 8;              // 16-byte chunks per K or V row
  static constexpr int ROW_BYTES = HD * 2;
  static constexpr int K_BYTES = BKV * HD * 2;    // K tile [64][HD], row-major
  static constexpr int V_BYTES = BKV * HD * 2;    // V tile [64][HD], row-major
  static constexpr int STAGE_BYTES = K_BYTES + V_BYTES;
  static constexpr int K_LOADS = K_BYTES / (NTHREADS * 16);  // DMA instructions per thread per tile
  static constexpr int V_LOADS = V_BYTES / (NTHREADS * 16);
  static constexpr int LOADS = K_LOADS + V_LOADS;
  static constexpr int ROWS_PER_LOAD = 64 / NCH;              // rows one wave instruction fills (1 KB)
  static constexpr int KK = HD / 16;                          // MFMA k-steps over head_dim
  static constexpr int DT = HD / 32;                          // 32-wide d tiles of O
  // V rows: the 16-byte chunk c of row r sits at c ^ ((r % 4) << VSH), which
  // moves the 64-byte (HD 128) or 32-byte (HD 64) pieces of the four rows of a
  // transposing read to four different bank ranges.
  static constexpr int VSH = HD == 128 ? 2 : 1;
  static_assert(K_LOADS >= 1 && V_LOADS >= 1, "tile too small for the workgroup");
  static_assert(HD == 64 || HD == 128, "head_dim 64 or 128");
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
  // The ring's stages are four distinct arrays, and every access names its
  // stage statically (the tile loops are unrolled by four): the compiler then
  // knows that a transposing read of one stage does not alias the DMA filling
  // another, and does not make it wait for every load in flight (it does when
  // they may alias, as for offsets into one array).
  __shared__ __attribute__((aligned(1024))) uint8_t stage0[C::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t stage1[C::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t stage2[C::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t stage3[C::STAGE_BYTES];
  static_assert(NSTAGE == 4, "one array per stage");
  // stage J (a compile-time constant) holds the tiles t_begin + J, + J + 4, ...
  auto stage_of = [&](auto J) __attribute__((always_inline)) -> uint8_t* {
    constexpr int j = decltype(J)::value & 3;
    if constexpr (j == 0) return stage0;
    else if constexpr (j == 1) return stage1;
    else if constexpr (j == 2) return stage2;
    else return stage3;
  };


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

  // ---- direct buffer->LDS loads.  Instruction i of wave w fills the 1 KB
  // block (i*NW + w) of the K (or V) region of a stage; lane L writes its 16
  // bytes at L*16: row r = block*ROWS_PER_LOAD + L/NCH, physical chunk L%NCH.
  // K: logical chunk (L % NCH) ^ (r % NCH).  V: (L % NCH) ^ ((r % 4) << VSH).
  // The byte offsets are relative to the tile's first key row at the head's
  // first column (the descriptors' base, rebased per tile).
  int k_row[C::K_LOADS], k_col[C::K_LOADS], v_row[C::V_LOADS], v_col[C::V_LOADS];
  uint32_t k_off[C::K_LOADS], v_off[C::V_LOADS];
#pragma unroll
  for (int i = 0; i < C::K_LOADS; ++i) {
    const int r = (i * NW + wave) * C::ROWS_PER_LOAD + lane / C::NCH;
    k_row[i] = r;
    k_col[i] = ((lane % C::NCH) ^ (r & (C::NCH - 1))) * 8;
    k_off[i] = (uint32_t)((r * kld + k_col[i]) * 2);
  }
#pragma unroll
  for (int i = 0; i < C::V_LOADS; ++i) {
    const int r = (i * NW + wave) * C::ROWS_PER_LOAD + lane / C::NCH;
    v_row[i] = r;
    v_col[i] = ((lane % C::NCH) ^ ((r & 3) << C::VSH)) * 8;
    v_off[i] = (uint32_t)((r * kld + v_col[i]) * 2);
  }
  const uint16_t* k_head = a.k + kcol;
  const uint16_t* v_head = a.v + kcol;

  // WHOLE: the caller knows that the tile lies inside the key range (no
  // branch on it).
  auto issue_tile = [&](int t, auto J, auto WHOLE) __attribute__((always_inline)) {
    uint8_t* stage = stage_of(J);
    const int64_t k0 = (int64_t)t * BKV;
    // bytes from the tile's first row (head column) to the end of the sequence
    const int64_t span = (a.seq_len - k0) * kld * 2 - (int64_t)kcol * 2;
    const uint32_t bytes = (uint32_t)min(span, (int64_t)0x7fffffff);
    const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(k_head + k0 * kld, bytes);
    const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(v_head + k0 * kld, bytes);
    if (decltype(WHOLE)::value || k0 + BKV <= key_end) {  // whole tile inside the key range (wave-uniform)
#pragma unroll
      for (int i = 0; i < C::K_LOADS; ++i) dma16_buf(rk, k_off[i], stage + (i * NW + wave) * 1024);
#pragma unroll
      for (int i = 0; i < C::V_LOADS; ++i) dma16_buf(rv, v_off[i], stage + C::K_BYTES + (i * NW + wave) * 1024);
    } else {  // last tile: rows past the range re-read the last key (masked, and zero weight)
#pragma unroll
      for (int i = 0; i < C::K_LOADS; ++i) {
        const int r = (int)min((int64_t)k_row[i], key_end - 1 - k0);
        dma16_buf(rk, (uint32_t)((r * kld + k_col[i]) * 2), stage + (i * NW + wave) * 1024);
      }
#pragma unroll
      for (int i = 0; i < C::V_LOADS; ++i) {
        const int r = (int)min((int64_t)v_row[i], key_end - 1 - k0);
        dma16_buf(rv, (uint32_t)((r * kld + v_col[i]) * 2), stage + C::K_BYTES + (i * NW + wave) * 1024);
      }
    }
  };

  // ---- fragment read addresses (bytes within a stage).  K row r = kb*32 + ql,
  // logical chunk 2*kk + half, physical chunk (2*kk + half) ^ (r % NCH):
  // address = (row base | ((half ^ r%NCH) << 4)) ^ (kk << 5).
  const uint32_t k_a0 = (uint32_t)ql * C::ROW_BYTES + ((uint32_t)(half ^ (ql & (C::NCH - 1))) << 4);
  // V: a V^T fragment (lane l: d = dt*32 + l%32, MFMA k values 8(l/32) .. +7
  // of a 16-key step, i.e. keys key_perm16(8(l/32) + j)) is two transposing
  // reads of four key rows each.  In 16-lane group g = l/16, lane 4m + q names
  // key row key_perm16(8(g/2) + m) (first read) or key_perm16(8(g/2) + 4 + m)
  // (second), columns dt*32 + 16(g%2) + 4q .. +3; both rows are = m (mod 4).
  // Physical byte of that piece: row*ROW_BYTES + ((chunk ^ (m << VSH)) * 16 +
  // 8(q%2) with chunk = 4dt + 2(g%2) + q/2, so d tile dt flips bit 6 and step
  // ks adds 16 rows.
  uint32_t vr_a, vr_b;
  {
    const int g = lane >> 4, m = (lane >> 2) & 3, q = lane & 3;
    const int ka = key_perm16(8 * (g >> 1) + m), kb = key_perm16(8 * (g >> 1) + 4 + m);
    const uint32_t piece = ((uint32_t)((2 * (g & 1) + (q >> 1)) ^ (m << C::VSH)) << 4) + (uint32_t)(q & 1) * 8;
    vr_a = C::K_BYTES + (uint32_t)ka * C::ROW_BYTES + piece;
    vr_b = C::K_BYTES + (uint32_t)kb * C::ROW_BYTES + piece;
  }

  // ---- running state: m = running reference max of the raw scores, l =
  // lane-partial sum of the probabilities, relative to the reference r (log2
  // units): a probability is 2^(s * scale_log2 - r).
  //   * fma form (|m * scale_log2| < 2^10): r = mc = fl(m * scale_log2) and
  //     the exponent is one fma, s * scale_log2 - mc rounded once.  mc differs
  //     from m * scale_log2 by d, at most half its ulp (2^-14): a factor 2^d
  //     common to every probability of the row, which cancels in O / l and is
  //     part of the stored normaliser.  The bound keeps d negligible where it
  //     does not cancel: the max's probability 2^d enters O rounded to bf16
  //     but l in fp32, a relative error of about d ln 2 (at most 2^-9 for a
  //     larger d), which matters in rows that one key dominates.
  //   * exact form (larger scores, as in a deep stack without a norm):
  //     r = m * scale_log2 and the exponent is (s - m) * scale_log2, whose
  //     difference is exact near the max, so the exponent of the max is
  //     exactly 0 at any magnitude.
  // The form is wave-uniform and only moves from fma to exact.
  constexpr float inv_sqrt_hd = HD == 128 ? 0.08838834764831844055f : 0.125f;
  const float scale_log2 = 1.44269504088896340736f * inv_sqrt_hd;
  const float tau_raw = LAZY_TAU / scale_log2;  // the rescale threshold in raw score units
  constexpr float FMA_LIMIT = 1024.0f;          // 2^10: |mc| below it keeps the fma form
  // A lane's 32 probabilities of a tile sum to at most 2^13 while none exceeds
  // 2^LAZY_TAU; above it (or non-finite) the fma form's tile is redone.
  constexpr float LSUM_MAX = 8192.0f;
  float m_run = -INFINITY;
  float mc = -INFINITY;  // fl(m_run * scale_log2)
  bool exact = false;    // wave-uniform
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

  // Raw row max of a tile's (masked) scores, combined over the lane pair
  // (lanes l and l+32 hold the two halves of a query's keys).
  auto tile_max = [&](f32x16 (&s)[2]) __attribute__((always_inline)) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kb][e]);
    return pair_max(mx);
  };

  // ---- ping-pong schedule.  Per tile t every wave runs two phases, each
  // ended by a workgroup barrier:
  //   softmax(t): mask (diagonal tiles), max, lazy rescale, exponentials and
  //               row sum of its scores S(t) -> P(t) as bf16 pairs (vector
  //               work); on the fast path the V(t) fragments of the first two
  //               16-key steps are then read into registers (tile t is
  //               visible since matmul(t-2));
  //   matmul(t):  load tile t+3, O += V(t)^T P(t) (on the fast path with the
  //               other V(t) fragment reads, then the K(t+1) reads, between
  //               its MFMA steps), S(t+1) = K(t+1) Q^T (32 MFMAs), then wait
  //               for this wave's loads of tile t+2.
  // Waves 4-7 pass one extra barrier before their first phase and waves 0-3
  // one after their last, so waves 4-7 run one phase behind waves 0-3: with
  // one wave of each group per SIMD, one wave's MFMAs run while the other's
  // vector work issues beside them.  Both groups run the same code.
  // Stage J of the ring holds tiles t_begin + J (mod 4).  Tile t+3 refills the
  // stage of tile t-1, whose last reader (a group-1 matmul(t-1)) ended before
  // a group-0 matmul(t) starts; tile t+1, read by matmul(t), was waited for by
  // every wave in its matmul(t-1), before the barrier that precedes a group-0
  // matmul(t).
  const int grp = wave >> 2;                     // one wave of each group per SIMD
  const int wave_last = min(wave_tiles, t_end);  // tiles t < wave_last are computed by this wave
  f32x16 s[2];      // scores S(t) of the wave's current tile
  uint32_t pk[16];  // P(t): bf16 pairs, pk[4*ks + j] holds keys of 16-key step ks

  // Probabilities of the scores s in the fma or the exact form -> pk, and
  // their lane sum.
  auto probs = [&](auto EXACT) __attribute__((always_inline)) {
    float lsum = 0.0f;
#pragma unroll
    for (int idx = 0; idx < 16; ++idx) {
      const int kb = idx >> 3, e = (2 * idx) & 15;
      float p0, p1;
      if constexpr (decltype(EXACT)::value) {
        p0 = __builtin_amdgcn_exp2f((s[kb][e] - m_run) * scale_log2);
        p1 = __builtin_amdgcn_exp2f((s[kb][e + 1] - m_run) * scale_log2);
      } else {
        p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][e], scale_log2, -mc));
        p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][e + 1], scale_log2, -mc));
      }
      lsum += p0 + p1;
      pk[idx] = pack_bf16x2(p0, p1);
    }
    return lsum;
  };

  // Softmax of tile t: in the fma form the probabilities are taken against
  // the current reference straight away, and the tile is redone only when a
  // lane's sum says that some score exceeds the reference by more than
  // 2^LAZY_TAU (a new max; the first tile, whose reference is -inf, always).
  // Redone, or in the exact form: the tile max, the lazy rescale (the
  // reference moves only when the max exceeds it by more than LAZY_TAU in
  // log2 units, so probabilities stay below 2^8), then the probabilities.
  auto softmax = [&](int t, auto masked) __attribute__((always_inline)) {
    if constexpr (decltype(masked)::value) mask_tile(t, s);
    float lsum = 0.0f;
    bool done = false;
    if (!exact) {
      lsum = probs(std::false_type{});
      done = __builtin_amdgcn_ballot_w64(!(lsum <= LSUM_MAX)) == 0;  // wave-uniform
    }
    if (!done) {  // rare in the fma form
      const float mt = tile_max(s);
      if (__builtin_amdgcn_ballot_w64(mt > m_run + tau_raw) != 0) {  // wave-uniform
        const float m_new = fmaxf(m_run, mt);
        const float mc_new = m_new * scale_log2;
        const bool exact_new = exact || __builtin_amdgcn_ballot_w64(!(fabsf(mc_new) < FMA_LIMIT)) != 0;
        // old reference -> new: exact m*c, or the rounded mc of the fma form
        float alpha;
        if (exact)
          alpha = __builtin_amdgcn_exp2f((m_run - m_new) * scale_log2);
        else if (exact_new)
          alpha = __builtin_amdgcn_exp2f(__builtin_fmaf(-m_new, scale_log2, mc));
        else
          alpha = __builtin_amdgcn_exp2f(mc - mc_new);
        m_run = m_new;
        mc = mc_new;
        exact = exact_new;
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) o[dt] *= alpha;
      }
      lsum = exact ? probs(std::true_type{}) : probs(std::false_type{});
    }
    l_run += lsum;
  };

  auto vfrag_at = [&](const uint8_t* vst, int dt, int ks) __attribute__((always_inline)) {
    const uint8_t* sb = vst + ks * 16 * C::ROW_BYTES;
    const u32x2 ra = lds_read_tr16x4(sb + (vr_a ^ (uint32_t)(dt << 6)));
    const u32x2 rb = lds_read_tr16x4(sb + (vr_b ^ (uint32_t)(dt << 6)));
    return u32x4{ra[0], ra[1], rb[0], rb[1]};
  };
  // V(t) fragments: steps 0, 1 read at the end of softmax(t), steps 2, 3 under
  // the first PV MFMAs.  All four in the softmax phase is faster at unit
  // scale but lengthens that phase where it is already the longer one (the
  // exact form, larger scores); half is as fast as either in both regimes.
  u32x4 vpre[4][C::DT];
  auto vload = [&](auto J) __attribute__((always_inline)) {
    const uint8_t* vst = stage_of(J);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) vpre[ks][dt] = vfrag_at(vst, dt, ks);
  };
  // Fast path: PV from stage J's V fragments (two steps already in
  // registers), with the remaining V reads and then the K(t+1) fragment reads
  // of stage JN spread between its MFMA steps, then S(t+1).
  auto matmul_fast = [&](auto J, auto JN) __attribute__((always_inline)) {
    const uint8_t* vst = stage_of(J);
    const uint8_t* kst = stage_of(JN);
    constexpr int KPS = 2 * C::KK / 2;  // K fragment reads per PV step (steps 2, 3)
    u32x4 kf[2 * C::KK];                // index 2*kk + kb
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 p = as_bf16x8(u32x4{pk[4 * ks], pk[4 * ks + 1], pk[4 * ks + 2], pk[4 * ks + 3]});
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) o[dt] = mfma32(as_bf16x8(vpre[ks][dt]), p, o[dt]);
      if (ks < 2) {  // V fragments of steps 2, 3
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) vpre[ks + 2][dt] = vfrag_at(vst, dt, ks + 2);
        __builtin_amdgcn_sched_group_barrier(0x008, C::DT, 0);    // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * C::DT, 0);  // DS read
      } else {
#pragma unroll
        for (int i = 0; i < KPS; ++i) {
          const int f = (ks - 2) * KPS + i, kk = f >> 1, kb = f & 1;
          kf[f] = *reinterpret_cast<const u32x4*>(kst + kb * 32 * C::ROW_BYTES + (k_a0 ^ (uint32_t)(kk << 5)));
        }
        __builtin_amdgcn_sched_group_barrier(0x008, C::DT, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, KPS, 0);    // DS read
      }
    }
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {
      s[0] = mfma32(as_bf16x8(kf[2 * kk]), qf[kk], s[0]);
      s[1] = mfma32(as_bf16x8(kf[2 * kk + 1]), qf[kk], s[1]);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * C::KK, 0);
  };
  // General path: O += V^T P from stage J (DT chains over the four 16-key
  // steps, V fragments one step ahead).
  auto pv = [&](auto J) __attribute__((always_inline)) {
    const uint8_t* vst = stage_of(J);
    auto vfrag = [&](int dt, int ks) __attribute__((always_inline)) { return vfrag_at(vst, dt, ks); };
    u32x4 v[C::DT];
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) v[dt] = vfrag(dt, 0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 w[C::DT];
      if (ks + 1 < 4) {
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) w[dt] = vfrag(dt, ks + 1);
      }
      const bf16x8 p = as_bf16x8(u32x4{pk[4 * ks], pk[4 * ks + 1], pk[4 * ks + 2], pk[4 * ks + 3]});
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) o[dt] = mfma32(as_bf16x8(v[dt]), p, o[dt]);
      if (ks + 1 < 4) {
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) v[dt] = w[dt];
      }
    }
  };
  // General path: S = K Q^T from stage J (two chains over the head_dim
  // steps, K fragments one step ahead).
  auto qk = [&](auto J) __attribute__((always_inline)) {
    const uint8_t* kst = stage_of(J);
    auto kfrag = [&](int kb, int kk) __attribute__((always_inline)) {
      return *reinterpret_cast<const u32x4*>(kst + kb * 32 * C::ROW_BYTES + (k_a0 ^ (uint32_t)(kk << 5)));
    };
    u32x4 a0 = kfrag(0, 0), a1 = kfrag(1, 0);
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {
      u32x4 b0 = a0, b1 = a1;
      if (kk + 1 < C::KK) {
        b0 = kfrag(0, kk + 1);
        b1 = kfrag(1, kk + 1);
      }
      s[0] = mfma32(as_bf16x8(a0), qf[kk], s[0]);
      s[1] = mfma32(as_bf16x8(a1), qf[kk], s[1]);
      a0 = b0;
      a1 = b1;
    }
  };

  // Phase boundary: no instruction moves across it.
  auto phase_end = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  using TT = std::true_type;
  using FT = std::false_type;
  // Both phases of tile t (stage J).  FAST: tile t needs no mask, the wave
  // computes tiles t and t+1, tiles t+1 .. t+3 lie inside the range and are
  // whole (no branch at all).
  auto tile_phases = [&](int t, auto J, auto FAST) __attribute__((always_inline)) {
    using JN = std::integral_constant<int, decltype(J)::value + 1>;
    using JL = std::integral_constant<int, decltype(J)::value + 3>;  // stage of tile t+3 (= t-1)
    if constexpr (decltype(FAST)::value) {
      softmax(t, FT{});
      vload(J);
      phase_end();
      issue_tile(t + NSTAGE - 1, JL{}, TT{});
      __builtin_amdgcn_s_setprio(1);  // this wave's MFMAs first, the other wave's vector work beside them
      matmul_fast(J, JN{});
      __builtin_amdgcn_s_setprio(0);
      wait_vmcnt<C::LOADS>();
      phase_end();
    } else {
      if (t < wave_last) softmax(t, TT{});
      phase_end();
      if (t + NSTAGE - 1 < t_end) issue_tile(t + NSTAGE - 1, JL{}, FT{});
      if (t < wave_last) {
        pv(J);
        if (t + 1 < wave_last) qk(JN{});
      }
      if (t + 2 < t_end) {
        if (t + 3 < t_end)
          wait_vmcnt<C::LOADS>();
        else
          wait_vmcnt<0>();
      }
      phase_end();
    }
  };

  using J0 = std::integral_constant<int, 0>;
  using J1 = std::integral_constant<int, 1>;
  using J2 = std::integral_constant<int, 2>;
  using J3 = std::integral_constant<int, 3>;

  // ---- prologue: tiles t_begin .. t_begin+NSTAGE-2 in flight, wait for the first.
  const int pro = max(min(NSTAGE - 1, t_end - t_begin), 0);
  if (pro > 0) issue_tile(t_begin, J0{}, FT{});
  if (pro > 1) issue_tile(t_begin + 1, J1{}, FT{});
  if (pro > 2) issue_tile(t_begin + 2, J2{}, FT{});
  if (pro >= 3)
    wait_vmcnt<2 * C::LOADS>();
  else if (pro == 2)
    wait_vmcnt<C::LOADS>();
  else
    wait_vmcnt<0>();
  lds_barrier();
  if (grp == 1) phase_end();  // group 1 runs one phase behind
  if (t_begin < wave_last) qk(J0{});
  if (t_begin + 1 < t_end) {  // tile t_begin+1, read by matmul(t_begin)
    if (t_begin + 2 < t_end)
      wait_vmcnt<C::LOADS>();
    else
      wait_vmcnt<0>();
  }
  phase_end();

  // Fast iterations: tiles t .. t+3 lie before the workgroup's first query
  // (no mask for any wave, and every active wave computes tiles up to t+4),
  // tiles up to t+6 are whole and inside [t_begin, t_end).  Waves without a
  // valid query take the general form, with the same barriers.  Iterations of
  // four tiles keep each tile's stage static.
  const int t_m = (int)((pos0 + 1) / BKV);  // first tile that some wave masks
  const int64_t key_lim = min(key_end, (int64_t)t_end * BKV);
  int t = t_begin;
  if (wave_active) {
    for (; t + 4 <= t_m && (int64_t)(t + 7) * BKV <= key_lim; t += 4) {
      tile_phases(t, J0{}, TT{});
      tile_phases(t + 1, J1{}, TT{});
      tile_phases(t + 2, J2{}, TT{});
      tile_phases(t + 3, J3{}, TT{});
    }
  } else {
    for (; t + 4 <= t_m && (int64_t)(t + 7) * BKV <= key_lim; t += 4) {
      tile_phases(t, J0{}, FT{});
      tile_phases(t + 1, J1{}, FT{});
      tile_phases(t + 2, J2{}, FT{});
      tile_phases(t + 3, J3{}, FT{});
    }
  }
  for (; t < t_end; t += 4) {
    tile_phases(t, J0{}, FT{});
    if (t + 1 < t_end) tile_phases(t + 1, J1{}, FT{});
    if (t + 2 < t_end) tile_phases(t + 2, J2{}, FT{});
    if (t + 3 < t_end) tile_phases(t + 3, J3{}, FT{});
  }
  if (grp == 0) phase_end();  // pairs with group 1's first extra barrier
  wait_vmcnt<0>();

  if (SPLIT && part >= 0) {
    // unnormalised output, running max (scaled to log2 units) and sum of this key half
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
        ml[0] = mc;  // the reference r (fl(m * scale_log2) in the exact form)
        ml[1] = l_tot;
      }
    }
    return;
  }

  // ---- normalise and store: lane holds query ql, dims dt*32 + 8*(e/4) + 4*half + e%4.
  if (wave_active) {
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (a.lse && half == 0 && wave_first + ql < valid)  // sum_j exp(s_j) = 2^r * l_tot
      a.lse[(int64_t)head * 2 * a.chunk_len + row0 + wave_first + ql] =
          (mc + log2f(l_tot)) * 0.69314718055994530942f;
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

}  // namespace

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

hipError_t launch_attention(const AttnArgs& args, hipStream_t stream) {
  if (args.chunk_len <= 0) return hipSuccess;
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
  // the key halves' partials in the workspace
  AttnArgs a = args;
  char* base = static_cast<char*>(a.ws);
  a.part_o = reinterpret_cast<float*>(base);
  a.part_ml = reinterpret_cast<float*>(base + attn_align((size_t)2 * a.chunk_len * a.hidden * 4));
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
